// Dispatch on one GPU: regroup the T*k (token, slot) assignments into contiguous
// per-expert rows (moe_ffn's dispatch, "Decoding Trillion-Parameter MoE LLMs", section
// "Routing: Top-K Experts Plus a Shared Expert"; across GPUs this is the all-to-all of
// the WideEP claim card's "Context After" paragraph). Rows are ordered by expert id,
// then by token, so the permutation is unique and the result deterministic.
//
// k_hist    one wavefront per block of 64 tokens: each lane ORs its bit into an LDS
//           64-bit mask per expert (ds_or_b64; order-free, so deterministic). The masks
//           and their popcounts (per-block counts) go to the workspace.
// k_scan    one workgroup: per-expert totals (each expert's blocks split into chunks over
//           the 1024 threads), exclusive scan over experts (offsets), then each block's
//           base row per expert; optionally the tile list for the grouped GEMM (row
//           chunks of tile_m rows per expert, plus the shared group).
// k_scatter one wavefront per block: row = base[block][e] + number of earlier tokens of
//           the block that chose e (popcount of the mask below the lane).
// k_gather  x_perm[r] = x[perm_src[r] / k], 16 B per lane.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kScanThreads = 1024;
#ifndef MOE_SCAN_UNROLL  // blocks whose counts one scan thread loads at once (1 -> 8:
#define MOE_SCAN_UNROLL 8   // k_scan 19.5 -> 12 us at e384_fp8)
#endif

__global__ void __launch_bounds__(64) k_hist(const int32_t* __restrict__ topk_idx, int T, int k,
                                             int E, uint64_t* __restrict__ masks,
                                             int32_t* __restrict__ cnt) {
  __shared__ uint64_t m[1024];
  const int l = threadIdx.x;
  const int b = blockIdx.x;
  for (int e = l; e < E; e += 64) m[e] = 0ull;
  __syncthreads();
  const int t = b * 64 + l;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = topk_idx[(int64_t)t * k + j];
      atomicOr(reinterpret_cast<unsigned long long*>(&m[e]), 1ull << l);
    }
  }
  __syncthreads();
  for (int e = l; e < E; e += 64) {
    masks[(int64_t)b * E + e] = m[e];
    cnt[(int64_t)b * E + e] = __popcll(m[e]);
  }
}

// Exclusive scan of v over the workgroup (kScanThreads threads); returns the prefix,
// total in *total.
__device__ int block_exclusive_scan(int v, int* sh, int* total) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int o = 1; o < kScanThreads; o <<= 1) {
    int add = tid >= o ? sh[tid - o] : 0;
    __syncthreads();
    sh[tid] += add;
    __syncthreads();
  }
  int incl = sh[tid];
  *total = sh[kScanThreads - 1];
  __syncthreads();
  return incl - v;
}

// Tile i of the nt tiles of group g (rows [row0, row0 + rows)), placed at index toff + i:
// tile_m-row chunks, in blocks of up to kTileBlock consecutive tiles.
__device__ Tile make_tile(int g, int row0, int rows, int i, int nt, int toff, int tile_m) {
  Tile tl;
  tl.group = g;
  tl.row0 = row0 + i * tile_m;
  tl.nrows = min(tile_m, rows - i * tile_m);
  const int b0 = i / kTileBlock * kTileBlock;
  tl.blk0 = toff + b0;
  tl.nblk = min(kTileBlock, nt - b0);
  tl.pad[0] = tl.pad[1] = tl.pad[2] = 0;
  return tl;
}

__global__ void __launch_bounds__(kScanThreads) k_scan(int32_t* __restrict__ cnt, int nb, int E,
                                                       int T, int k, int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ offsets,
                                                       Tile* __restrict__ tiles,
                                                       int32_t* __restrict__ ntiles, int tile_m,
                                                       int with_shared) {
  __shared__ int sh[kScanThreads];
  __shared__ int part_sum[kScanThreads];
  // Thread tid works on expert tid % E and on part tid / E of that expert's blocks: P
  // contiguous chunks of C blocks, so that the per-block counts of one expert are summed
  // and turned into running bases by P threads instead of one.
  const int tid = threadIdx.x;
  const int P = E <= kScanThreads ? kScanThreads / E : 1;
  const int C = (nb + P - 1) / P;
  const int pe = tid % E, part = tid / E;
  const bool worker = part < P;
  const int b0 = part * C, b1 = min(nb, b0 + C);
  int s = 0;
  if (worker) {
#pragma unroll MOE_SCAN_UNROLL
    for (int b = b0; b < b1; ++b) s += cnt[(int64_t)b * E + pe];
  }
  part_sum[tid] = worker ? s : 0;
  __syncthreads();
  // per expert: exclusive prefix over its parts, and its total
  int pre = 0, tot_pe = 0;
  if (worker)
    for (int q = 0; q < P; ++q) {
      const int v = part_sum[q * E + pe];
      if (q < part) pre += v;
      tot_pe += v;
    }
  // expert offsets: exclusive scan over experts (threads tid < E hold part 0)
  const int e = tid;
  const int tot = (e < E) ? tot_pe : 0;
  int all;
  const int off = block_exclusive_scan(tot, sh, &all);
  // off of expert pe, as seen by every part of it
  __syncthreads();
  if (e < E) sh[e] = off;
  __syncthreads();
  if (worker) {
    int run = sh[pe] + pre;
#pragma unroll MOE_SCAN_UNROLL
    for (int b = b0; b < b1; ++b) {
      const int c = cnt[(int64_t)b * E + pe];
      cnt[(int64_t)b * E + pe] = run;
      run += c;
    }
  }
  if (e < E) {
    counts[e] = tot;
    offsets[e] = off;
  }
  if (e == 0) offsets[E] = all;
  __syncthreads();  // every part has read its expert's offset from sh before sh is reused
  if (tiles) {
    // routed groups: ceil(count / tile_m) tiles each; the shared group E holds T rows
    // starting at row T*k
    int nt = 0, rows = 0, row0 = 0;
    if (e < E) { rows = tot; row0 = off; }
    else if (e == E && with_shared) { rows = T; row0 = T * k; }
    nt = (rows + tile_m - 1) / tile_m;
    int ntot;
    const int toff = block_exclusive_scan(nt, sh, &ntot);
    for (int i = 0; i < nt; ++i) tiles[toff + i] = make_tile(e, row0, rows, i, nt, toff, tile_m);
    if (e == 0) *ntiles = ntot;
  }
}

__global__ void __launch_bounds__(64) k_scatter(const int32_t* __restrict__ topk_idx, int T, int k,
                                                int E, const uint64_t* __restrict__ masks,
                                                const int32_t* __restrict__ base,
                                                int32_t* __restrict__ perm_src,
                                                int32_t* __restrict__ inv_perm,
                                                int32_t* __restrict__ row_token) {
  const int l = threadIdx.x;
  const int b = blockIdx.x;
  const int t = b * 64 + l;
  if (t >= T) return;
  const uint64_t below = (l == 0) ? 0ull : (~0ull >> (64 - l));
  for (int j = 0; j < k; ++j) {
    const int64_t a = (int64_t)t * k + j;
    const int e = topk_idx[a];
    const uint64_t mk = masks[(int64_t)b * E + e];
    const int r = base[(int64_t)b * E + e] + __popcll(mk & below);
    perm_src[r] = (int32_t)a;
    inv_perm[a] = r;
    if (row_token) row_token[r] = t;
  }
}

// Rows of T*k .. T*k+T-1 (the shared group) read token r - T*k.
__global__ void k_shared_rows(int32_t* __restrict__ row_token, int T, int k) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < T) row_token[(int64_t)T * k + i] = i;
}

// The shared expert's group on its own: row_token of rows T*k .. T*k + T - 1 (token i at
// row T*k + i) and the tile list of that one group (group E), for a grouped-FFN launch that
// runs beside the routed one.
__global__ void k_shared_group(int32_t* __restrict__ row_token, int T, int k, int E, int tile_m,
                               Tile* __restrict__ tiles, int32_t* __restrict__ ntiles) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int nt = (T + tile_m - 1) / tile_m;
  if (i < T) row_token[(int64_t)T * k + i] = i;
  if (i < nt) tiles[i] = make_tile(E, T * k, T, i, nt, 0, tile_m);
  if (i == 0) *ntiles = nt;
}

__global__ void __launch_bounds__(256) k_gather(const uint4* __restrict__ x, int vec_per_row,
                                                const int32_t* __restrict__ perm_src, int k,
                                                int rows, uint4* __restrict__ xp) {
  const int r = blockIdx.x;
  const int src = perm_src[r] / k;
  for (int v = blockIdx.y * 256 + threadIdx.x; v < vec_per_row; v += gridDim.y * 256)
    xp[(int64_t)r * vec_per_row + v] = x[(int64_t)src * vec_per_row + v];
}

__global__ void __launch_bounds__(kScanThreads) k_tiles_from_offsets(const int32_t* __restrict__ offsets,
                                                                     int E, Tile* __restrict__ tiles,
                                                                     int32_t* __restrict__ ntiles,
                                                                     int tile_m) {
  __shared__ int sh[kScanThreads];
  const int e = threadIdx.x;
  int rows = 0, row0 = 0;
  if (e < E) {
    row0 = offsets[e];
    rows = offsets[e + 1] - row0;
  }
  const int nt = (rows + tile_m - 1) / tile_m;
  int ntot;
  const int toff = block_exclusive_scan(nt, sh, &ntot);
  for (int i = 0; i < nt; ++i) tiles[toff + i] = make_tile(e, row0, rows, i, nt, toff, tile_m);
  if (e == 0) *ntiles = ntot;
}

// Two tile lists from the offsets: groups with more than cold_max rows ("hot": many rows
// per expert, the tiled kernels' work) in tm_hot-row tiles, groups with 1..cold_max rows
// ("cold": their weights stream, few rows to multiply) in tm_cold-row tiles. The shared
// group E (T rows at row T*k), when present, is classified the same way.
__global__ void __launch_bounds__(kScanThreads) k_split_tiles(const int32_t* __restrict__ offsets,
                                                              int E, int T, int k, int with_shared,
                                                              int cold_max, int tm_hot,
                                                              Tile* __restrict__ hot,
                                                              int32_t* __restrict__ n_hot,
                                                              int tm_cold, Tile* __restrict__ cold,
                                                              int32_t* __restrict__ n_cold) {
  __shared__ int sh[kScanThreads];
  const int e = threadIdx.x;
  int rows = 0, row0 = 0;
  if (e < E) {
    row0 = offsets[e];
    rows = offsets[e + 1] - row0;
  } else if (e == E && with_shared) {
    row0 = T * k;
    rows = T;
  }
  const bool is_cold = rows <= cold_max;
  const int nh = is_cold ? 0 : (rows + tm_hot - 1) / tm_hot;
  const int nc = is_cold ? (rows + tm_cold - 1) / tm_cold : 0;
  int th, tc;
  const int oh = block_exclusive_scan(nh, sh, &th);
  const int oc = block_exclusive_scan(nc, sh, &tc);
  for (int i = 0; i < nh; ++i) hot[oh + i] = make_tile(e, row0, rows, i, nh, oh, tm_hot);
  for (int i = 0; i < nc; ++i) cold[oc + i] = make_tile(e, row0, rows, i, nc, oc, tm_cold);
  if (e == 0) {
    *n_hot = th;
    *n_cold = tc;
  }
}

}  // namespace

size_t permute_ws_bytes(int32_t T, int32_t E) {
  const size_t nb = (size_t)(T + 63) / 64;
  size_t masks = nb * E * sizeof(uint64_t);
  size_t cnt = nb * E * sizeof(int32_t);
  return (masks + 255) / 256 * 256 + (cnt + 255) / 256 * 256;
}

hipError_t launch_permute_maps(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                               int32_t* counts, int32_t* offsets, int32_t* perm_src,
                               int32_t* inv_perm, int32_t* row_token, Tile* tiles,
                               int32_t* ntiles, int32_t tile_m, int32_t with_shared, void* ws,
                               hipStream_t s) {
  const int nb = (T + 63) / 64;
  uint64_t* masks = reinterpret_cast<uint64_t*>(ws);
  size_t mbytes = ((size_t)nb * E * sizeof(uint64_t) + 255) / 256 * 256;
  int32_t* cnt = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + mbytes);
  if (nb > 0) {
    hipLaunchKernelGGL(k_hist, dim3(nb), dim3(64), 0, s, topk_idx, T, k, E, masks, cnt);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(kScanThreads), 0, s, cnt, nb, E, T, k, counts, offsets,
                     tiles, ntiles, tile_m, with_shared);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (nb > 0) {
    hipLaunchKernelGGL(k_scatter, dim3(nb), dim3(64), 0, s, topk_idx, T, k, E, masks, cnt, perm_src,
                       inv_perm, row_token);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (row_token && with_shared && T > 0) {
    hipLaunchKernelGGL(k_shared_rows, dim3((T + 255) / 256), dim3(256), 0, s, row_token, T, k);
    err = hipGetLastError();
  }
  return err;
}

hipError_t launch_gather_rows(const void* x, int32_t elem_bytes, int32_t H,
                              const int32_t* perm_src, int32_t k, int32_t rows, void* x_perm,
                              hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int vec = (int)((int64_t)H * elem_bytes / 16);
  const int gx = (vec + 255) / 256;
  hipLaunchKernelGGL(k_gather, dim3(rows, gx), dim3(256), 0, s, reinterpret_cast<const uint4*>(x),
                     vec, perm_src, k, rows, reinterpret_cast<uint4*>(x_perm));
  return hipGetLastError();
}

hipError_t launch_shared_group(int32_t T, int32_t k, int32_t E, int32_t tile_m, int32_t* row_token,
                               Tile* tiles, int32_t* ntiles, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_shared_group, dim3((T + 255) / 256), dim3(256), 0, s, row_token, T, k, E,
                     tile_m, tiles, ntiles);
  return hipGetLastError();
}

hipError_t launch_split_tiles(const int32_t* offsets, int32_t E, int32_t T, int32_t k,
                              int32_t with_shared, int32_t cold_max, int32_t tm_hot, Tile* hot,
                              int32_t* n_hot, int32_t tm_cold, Tile* cold, int32_t* n_cold,
                              hipStream_t s) {
  hipLaunchKernelGGL(k_split_tiles, dim3(1), dim3(kScanThreads), 0, s, offsets, E, T, k,
                     with_shared, cold_max, tm_hot, hot, n_hot, tm_cold, cold, n_cold);
  return hipGetLastError();
}

hipError_t launch_tiles_from_offsets(const int32_t* offsets, int32_t E, Tile* tiles,
                                     int32_t* ntiles, int32_t tile_m, hipStream_t s) {
  hipLaunchKernelGGL(k_tiles_from_offsets, dim3(1), dim3(kScanThreads), 0, s, offsets, E, tiles,
                     ntiles, tile_m);
  return hipGetLastError();
}

}  // namespace moe
