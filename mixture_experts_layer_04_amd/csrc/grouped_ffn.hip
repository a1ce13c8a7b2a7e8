// Grouped SwiGLU expert FFN: for every expert (group), h = SiLU(x Wg^T) * (x Wu^T) on its
// rows, then y = h W2^T -- the per-expert FFN of moe_ffn ("Decoding Trillion-Parameter
// MoE LLMs", section "Routing: Top-K Experts Plus a Shared Expert") run as one grouped
// GEMM pair with SwiGLU fused into the gate/up epilogue, as in the grouped GEMM of
// "GC-MoE: Overlapping Expert-Parallel Token Dispatch with FP8/FP4 Grouped GEMM via CUDA
// Green Contexts" (key_changes, fourth item). Decode is bound by streaming the weights of
// the touched experts ("why_it_matters" of the same record).
//
// Work is described by a device-side tile list (permute.hip): each tile is up to tile_m
// rows of one group. Launch grids use a host-side upper bound on the tile count; surplus
// workgroups exit at once, so no host synchronisation is needed.
//
// Streaming kernels (few rows per expert, e.g. decode): the weights are the MFMA A
// operand (16 output features per wavefront), the <= 16 rows of the tile the B operand.
// Each lane loads 32 contiguous bytes of its weight row per step (a full 128 B line per
// 4 lanes), straight from HBM into registers with non-temporal loads: a weight element
// is read exactly once per tile and never staged in LDS. bf16 uses
// v_mfma_f32_16x16x32_bf16, fp32 v_mfma_f32_16x16x4_f32. Because a dot product may be
// summed in any order, the K index carried by lane group kq and register slot j is
// k0 + 16*kq + j (bf16) -- the same map for A and B -- which makes every load contiguous.
#include "moe_internal.h"

namespace moe {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kStreamTileM = 16;
constexpr int kFeatPerWG = 64;  // 4 wavefronts x 16 output features

struct Frag32 {  // 32 bytes per lane
  u32x4 lo, hi;
};

__device__ __forceinline__ Frag32 load_nt(const void* p) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
  Frag32 f;
  f.lo = __builtin_nontemporal_load(q);
  f.hi = __builtin_nontemporal_load(q + 1);
  return f;
}
__device__ __forceinline__ Frag32 load_c(const void* p) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
  Frag32 f;
  f.lo = q[0];
  f.hi = q[1];
  return f;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// acc += A(32 B of bf16) x B(32 B of bf16): two 16x16x32 MFMAs
__device__ __forceinline__ f32x4 mma_bf16(const Frag32& a, const Frag32& b, f32x4 acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a.lo), as_bf16x8(b.lo), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a.hi), as_bf16x8(b.hi), acc, 0, 0, 0);
  return acc;
}
// acc += A(8 fp32) x B(8 fp32): eight 16x16x4 MFMAs, register slot j carries k = base + j
__device__ __forceinline__ f32x4 mma_f32(const Frag32& a, const Frag32& b, f32x4 acc) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.lo[j]), __uint_as_float(b.lo[j]),
                                              acc, 0, 0, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.hi[j]), __uint_as_float(b.hi[j]),
                                              acc, 0, 0, 0);
  return acc;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

template <bool kF32>
__device__ __forceinline__ void store4(void* base, int64_t off, f32x4 v) {
  if (kF32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + off) =
        make_float4(v[0], v[1], v[2], v[3]);
  } else {
    uint2 p;
    p.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    p.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(base) + off) = p;
  }
}

// Tuning constants of the streaming kernels (K steps per loop iteration, weight load
// cache policy). Weights are read with ordinary cached loads: on MI355X they measured
// faster than non-temporal ones for this many-rows-at-once access pattern.
#ifndef MOE_STREAM_UNROLL_GU
#define MOE_STREAM_UNROLL_GU 4
#endif
#ifndef MOE_STREAM_UNROLL_DN
#define MOE_STREAM_UNROLL_DN 8
#endif
#ifndef MOE_STREAM_NT
#define MOE_STREAM_NT 0
#endif

__device__ __forceinline__ Frag32 load_w(const void* p) {
  return MOE_STREAM_NT ? load_nt(p) : load_c(p);
}
// Activation fragment of a row; lanes of padding rows (beyond the tile's rows) load
// nothing and contribute zeros to columns that are never stored.
__device__ __forceinline__ Frag32 load_x(const void* p, bool valid) {
  if (valid) return load_c(p);
  Frag32 z;
  z.lo = u32x4{0, 0, 0, 0};
  z.hi = u32x4{0, 0, 0, 0};
  return z;
}

template <bool kF32>
__device__ __forceinline__ f32x4 mma(const Frag32& w, const Frag32& x, f32x4 acc) {
  return kF32 ? mma_f32(w, x, acc) : mma_bf16(w, x, acc);
}

// Gate/up + SwiGLU. Workgroup = (tile, block of 64 h features); wavefront w computes
// features [f0, f0+16) of h: gate rows f0.. and up rows I+f0.. of W13[e].
template <bool kF32>
__global__ void __launch_bounds__(256) k_gateup_stream(FfnArgs a, int fb_per_tile) {
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int tile_id = blockIdx.x / fb_per_tile;
  const int fb = blockIdx.x - tile_id * fb_per_tile;
  if (tile_id >= *a.ntiles) return;
  const Tile tl = a.tiles[tile_id];
  const int bank = tl.group < a.E ? 0 : 1;
  const int64_t ge = tl.group < a.E ? tl.group : 0;
  const int I = a.bank[bank].I;
  const int H = a.H;
  const int f0 = fb * kFeatPerWG + wave * 16;
  if (f0 >= I) return;
  const int m = l & 15, kq = l >> 4;
  const int esz = kF32 ? 4 : 2;
  const char* w13 = reinterpret_cast<const char*>(a.bank[bank].w13) + ge * 2 * I * (int64_t)H * esz;
  const bool xv = m < tl.nrows;
  const int row = tl.row0 + (xv ? m : 0);
  const int64_t src = a.a_rowmap ? a.a_rowmap[row] : row;
  constexpr int kStep = kF32 ? 32 : 64;          // K elements per MFMA step
  constexpr int kLane = kStep / 4;               // contiguous elements per lane per step
  constexpr int U = MOE_STREAM_UNROLL_GU;
  const int64_t lane_off = (int64_t)kq * kLane * esz;
  const char* wg = w13 + (int64_t)(f0 + m) * H * esz + lane_off;
  const char* wu = w13 + (int64_t)(I + f0 + m) * H * esz + lane_off;
  const char* xr = reinterpret_cast<const char*>(a.a) + src * H * esz + lane_off;
  f32x4 accg = {0, 0, 0, 0}, accu = {0, 0, 0, 0};
  const int kmain = H - H % (kStep * U);
  for (int k0 = 0; k0 < kmain; k0 += kStep * U) {
    Frag32 fg[U], fu[U], fx[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t o = (int64_t)(k0 + u * kStep) * esz;
      fg[u] = load_w(wg + o);
      fu[u] = load_w(wu + o);
      fx[u] = load_x(xr + o, xv);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      accg = mma<kF32>(fg[u], fx[u], accg);
      accu = mma<kF32>(fu[u], fx[u], accu);
    }
  }
  for (int k0 = kmain; k0 < H; k0 += kStep) {
    const int64_t o = (int64_t)k0 * esz;
    Frag32 fg = load_w(wg + o), fu = load_w(wu + o), fx = load_x(xr + o, xv);
    accg = mma<kF32>(fg, fx, accg);
    accu = mma<kF32>(fu, fx, accu);
  }
  if (xv) {
    f32x4 hv;
#pragma unroll
    for (int i = 0; i < 4; ++i) hv[i] = silu_mul(accg[i], accu[i]);
    store4<kF32>(a.h, (int64_t)(tl.row0 + m) * a.I_max + f0 + kq * 4, hv);
  }
}

// Down projection. Workgroup = (tile, block of 64 output features of H).
template <bool kF32, bool kYF32>
__global__ void __launch_bounds__(256) k_down_stream(FfnArgs a, int fb_per_tile) {
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int tile_id = blockIdx.x / fb_per_tile;
  const int fb = blockIdx.x - tile_id * fb_per_tile;
  if (tile_id >= *a.ntiles) return;
  const Tile tl = a.tiles[tile_id];
  const int bank = tl.group < a.E ? 0 : 1;
  const int64_t ge = tl.group < a.E ? tl.group : 0;
  const int I = a.bank[bank].I;
  const int H = a.H;
  const int f0 = fb * kFeatPerWG + wave * 16;
  if (f0 >= H) return;
  const int m = l & 15, kq = l >> 4;
  const int esz = kF32 ? 4 : 2;
  constexpr int kStep = kF32 ? 32 : 64;
  constexpr int kLane = kStep / 4;
  constexpr int U = MOE_STREAM_UNROLL_DN;
  const int64_t lane_off = (int64_t)kq * kLane * esz;
  const bool xv = m < tl.nrows;
  const char* w2 = reinterpret_cast<const char*>(a.bank[bank].w2) + ge * (int64_t)H * I * esz;
  const char* wr = w2 + (int64_t)(f0 + m) * I * esz + lane_off;
  const char* hr = reinterpret_cast<const char*>(a.h) +
                   (int64_t)(tl.row0 + (xv ? m : 0)) * a.I_max * esz + lane_off;
  f32x4 acc = {0, 0, 0, 0};
  const int kmain = I - I % (kStep * U);
  for (int k0 = 0; k0 < kmain; k0 += kStep * U) {
    Frag32 fw[U], fh[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t o = (int64_t)(k0 + u * kStep) * esz;
      fw[u] = load_w(wr + o);
      fh[u] = load_x(hr + o, xv);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc = mma<kF32>(fw[u], fh[u], acc);
  }
  for (int k0 = kmain; k0 < I; k0 += kStep) {
    const int64_t o = (int64_t)k0 * esz;
    acc = mma<kF32>(load_w(wr + o), load_x(hr + o, xv), acc);
  }
  if (xv) store4<kYF32>(a.y, (int64_t)(tl.row0 + m) * H + f0 + kq * 4, acc);
}

// ---------------------------------------------------------------------------------
// Tiled kernels (many rows per expert, e.g. prefill): classic LDS-staged GEMM tiles of
// 128 rows x 128 weight rows x 64 K per workgroup, 4 wavefronts of 64 x 64 each built
// from v_mfma_f32_16x16x32_bf16. Global -> register prefetch of the next K block overlaps
// the MFMAs on the current one (double-buffered LDS, one barrier per K block). LDS rows are
// padded by 16 B so the 16-B fragment reads of 16 consecutive rows hit distinct banks.
// For gate/up, the 128 weight rows of a tile are 64 gate and the matching 64 up rows,
// interleaved in groups of 16 so that every lane holds gate and up of the same
// (row, feature) and SwiGLU is applied in registers.
constexpr int kTBM = 128, kTBN = 128, kTBK = 64;
constexpr int kLdsRow = kTBK * 2 + 16;                    // bytes per LDS row
constexpr int kLdsStage = (kTBM + kTBN) * kLdsRow;        // bytes per stage

// Workgroup id remap so that consecutive logical ids run on the same XCD (ids are dealt
// to the 8 XCDs round-robin), letting neighbours share their A tile in that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int grid) {
  if (grid % 8) return bid;
  return (bid % 8) * (grid / 8) + bid / 8;
}

template <bool kGateUp, bool kYF32>
__global__ void __launch_bounds__(256, 2) k_tiled_bf16(FfnArgs a, int nb_per_tile) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kLdsStage];
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int tile_id = bid / nb_per_tile;
  const int nb = bid - tile_id * nb_per_tile;
  if (tile_id >= *a.ntiles) return;
  const Tile tl = a.tiles[tile_id];
  const int bank = tl.group < a.E ? 0 : 1;
  const int64_t ge = tl.group < a.E ? tl.group : 0;
  const int I = a.bank[bank].I;
  const int H = a.H;
  const int K = kGateUp ? H : I;
  const int fpb = kGateUp ? kTBN / 2 : kTBN;              // output features per tile
  const int f0 = nb * fpb;
  if (f0 >= (kGateUp ? I : H)) return;
  const char* wbase = kGateUp
      ? reinterpret_cast<const char*>(a.bank[bank].w13) + ge * 2 * (int64_t)I * H * 2
      : reinterpret_cast<const char*>(a.bank[bank].w2) + ge * (int64_t)H * I * 2;
  // global -> LDS assignment: 16-B chunk c = tid + 256 i of a 128 x 128 B block
  const char* ag[4];
  const char* bg[4];
  int lds_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    const int r = c >> 3, col = (c & 7) * 16;
    lds_off[i] = r * kLdsRow + col;
    const int grow = tl.row0 + (r < tl.nrows ? r : tl.nrows - 1);
    if (kGateUp) {
      const int64_t src = a.a_rowmap ? a.a_rowmap[grow] : grow;
      ag[i] = reinterpret_cast<const char*>(a.a) + src * (int64_t)H * 2 + col;
      const int half = r >> 6, jj = r & 63, grp = jj >> 4, within = jj & 15;
      const int feat = f0 + half * 32 + (grp >> 1) * 16 + within;
      const int wrow = (grp & 1) ? I + feat : feat;
      bg[i] = wbase + (int64_t)wrow * K * 2 + col;
    } else {
      ag[i] = reinterpret_cast<const char*>(a.h) + (int64_t)grow * a.I_max * 2 + col;
      bg[i] = wbase + (int64_t)(f0 + r) * K * 2 + col;
    }
  }
  const int wm = wave & 1, wn = wave >> 1;
  const int m16 = l & 15, g = l >> 4;
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
  u32x4 ra[4], rb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ra[i] = *reinterpret_cast<const u32x4*>(ag[i]);
    rb[i] = *reinterpret_cast<const u32x4*>(bg[i]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    *reinterpret_cast<u32x4*>(smem + lds_off[i]) = ra[i];
    *reinterpret_cast<u32x4*>(smem + kTBM * kLdsRow + lds_off[i]) = rb[i];
  }
  __syncthreads();
  const int KT = K / kTBK;
  for (int kt = 0; kt < KT; ++kt) {
    const char* cur = smem + (kt & 1) * kLdsStage;
    if (kt + 1 < KT) {
      const int64_t o = (int64_t)(kt + 1) * kTBK * 2;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ra[i] = *reinterpret_cast<const u32x4*>(ag[i] + o);
        rb[i] = *reinterpret_cast<const u32x4*>(bg[i] + o);
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 fa[4], fb[4];
      const int kb = g * 32 + ks * 16;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        fa[t] = *reinterpret_cast<const bf16x8*>(cur + (wm * 64 + t * 16 + m16) * kLdsRow + kb);
        fb[t] = *reinterpret_cast<const bf16x8*>(cur + kTBM * kLdsRow +
                                                 (wn * 64 + t * 16 + m16) * kLdsRow + kb);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) {
      char* nxt = smem + ((kt + 1) & 1) * kLdsStage;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<u32x4*>(nxt + lds_off[i]) = ra[i];
        *reinterpret_cast<u32x4*>(nxt + kTBM * kLdsRow + lds_off[i]) = rb[i];
      }
    }
    __syncthreads();
  }
  // epilogue: lane holds D[row 4g+i][column m16] of each 16 x 16 sub-tile
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rl = wm * 64 + mt * 16 + 4 * g + i;
      if (rl >= tl.nrows) continue;
      const int64_t row = tl.row0 + rl;
      if (kGateUp) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int feat = f0 + wn * 32 + p * 16 + m16;
          const float hv = silu_mul(acc[mt][2 * p][i], acc[mt][2 * p + 1][i]);
          reinterpret_cast<uint16_t*>(a.h)[row * a.I_max + feat] = f32_to_bf16(hv);
        }
      } else {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const int64_t o = row * H + f0 + wn * 64 + nt * 16 + m16;
          if (kYF32) reinterpret_cast<float*>(a.y)[o] = acc[mt][nt][i];
          else reinterpret_cast<uint16_t*>(a.y)[o] = f32_to_bf16(acc[mt][nt][i]);
        }
      }
    }
  }
}

}  // namespace

int32_t ffn_tile_m(moe_dtype wdt, int32_t rows, int32_t groups, int32_t H) {
  // Few rows per expert: stream the weights (each weight element read once per tile of
  // <= 16 rows). Many rows: LDS-tiled GEMM with 128-row tiles.
  if (wdt == MOE_BF16 && H % kTBN == 0 && (int64_t)rows > 32 * (int64_t)groups) return kTBM;
  return kStreamTileM;
}

size_t ffn_scratch_bytes(moe_dtype wdt, int32_t rows_total, int32_t H, int32_t I_max) {
  (void)H;
  const size_t hb = (wdt == MOE_F32) ? 4 : 2;
  return ((size_t)rows_total * I_max * hb + 255) / 256 * 256;
}

hipError_t launch_grouped_ffn(FfnArgs a, void* scratch, hipStream_t s, hipEvent_t mid_event) {
  if (a.max_tiles <= 0) {
    return mid_event ? hipEventRecord(mid_event, s) : hipSuccess;
  }
  a.h = scratch;
  const int fb_gu = (a.I_max + kFeatPerWG - 1) / kFeatPerWG;
  const int fb_dn = (a.H + kFeatPerWG - 1) / kFeatPerWG;
  const bool f32 = a.wdt == MOE_F32;
  const bool yf32 = a.y_dt == MOE_F32;
  dim3 blk(256);
  if (a.tile_m == kTBM) {
    const int nb_gu = a.I_max / (kTBN / 2), nb_dn = a.H / kTBN;
    hipLaunchKernelGGL((k_tiled_bf16<true, false>), dim3(a.max_tiles * nb_gu), blk, 0, s, a, nb_gu);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (mid_event && (err = hipEventRecord(mid_event, s)) != hipSuccess) return err;
    if (yf32)
      hipLaunchKernelGGL((k_tiled_bf16<false, true>), dim3(a.max_tiles * nb_dn), blk, 0, s, a, nb_dn);
    else
      hipLaunchKernelGGL((k_tiled_bf16<false, false>), dim3(a.max_tiles * nb_dn), blk, 0, s, a, nb_dn);
    return hipGetLastError();
  }
  if (f32)
    hipLaunchKernelGGL(k_gateup_stream<true>, dim3(a.max_tiles * fb_gu), blk, 0, s, a, fb_gu);
  else
    hipLaunchKernelGGL(k_gateup_stream<false>, dim3(a.max_tiles * fb_gu), blk, 0, s, a, fb_gu);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (mid_event && (err = hipEventRecord(mid_event, s)) != hipSuccess) return err;
  if (f32 && yf32)
    hipLaunchKernelGGL((k_down_stream<true, true>), dim3(a.max_tiles * fb_dn), blk, 0, s, a, fb_dn);
  else if (f32)
    hipLaunchKernelGGL((k_down_stream<true, false>), dim3(a.max_tiles * fb_dn), blk, 0, s, a, fb_dn);
  else if (yf32)
    hipLaunchKernelGGL((k_down_stream<false, true>), dim3(a.max_tiles * fb_dn), blk, 0, s, a, fb_dn);
  else
    hipLaunchKernelGGL((k_down_stream<false, false>), dim3(a.max_tiles * fb_dn), blk, 0, s, a, fb_dn);
  return hipGetLastError();
}

hipError_t launch_quant_rows_fp8(const void*, int32_t, int32_t, uint8_t*, float*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace moe
