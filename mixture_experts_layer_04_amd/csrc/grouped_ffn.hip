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
// Tiled kernels (many rows per expert, e.g. prefill): LDS-staged GEMM tiles of
// BM = 32*TM rows x BN = 32*TN weight rows x 64 K per workgroup, 4 wavefronts in a 2 x 2
// grid, each computing (16*TM) x (16*TN) with v_mfma_f32_16x16x32_bf16. Global ->
// register prefetch of the next K block overlaps the MFMAs on the current one
// (double-buffered LDS, one barrier per K block). The LDS layout is the row-interleaved,
// XOR-swizzled one of lds_off(), which serves 16-row fragment reads at the full LDS rate.
// This kernel carries the MXFP4 weights; bf16 weights use the DMA kernel k_tiled2 below.
// A lane's fragment of a K block
// is the 32 contiguous bytes at 32*(lane/16) (K index = 16*(lane/16) + 8*ks + j in both
// operands). For gate/up, the BN weight rows of a tile are BN/2 gate rows and the matching
// BN/2 up rows, interleaved in groups of 16, so that each lane holds gate and up of the
// same (row, feature) and SwiGLU is applied in registers.
// MXFP4 weights: each thread converts its 8 E2M1 values (4 bytes) with their E8M0 block
// scale to bf16 on the way into LDS (v_cvt_scalef32_pk_bf16_fp4, exact), so the MFMA
// loop is the bf16 one.
#ifndef MOE_TILED_TM
#define MOE_TILED_TM 4
#endif
#ifndef MOE_TILED_TN
#define MOE_TILED_TN 4
#endif
constexpr int kTTM = MOE_TILED_TM, kTTN = MOE_TILED_TN;
constexpr int kTBM = 32 * kTTM, kTBN = 32 * kTTN, kTBK = 64;

__device__ __forceinline__ float e8m0_f32(uint32_t c) {
  if (c == 0xFFu) return __uint_as_float(0x7FC00000u);
  if (c == 0u) return __uint_as_float(0x00400000u);  // 2^-127
  return __uint_as_float(c << 23);
}

// LDS byte offset of logical 16-B chunk c of tile row r (each 16-row group takes
// eight 256-B lines, row j and row 8 + j share line j, chunks XOR-swizzled by row & 7;
// see the DMA kernel below).
__device__ __forceinline__ int lds_off(int r, int c) {
  return (r >> 4) * 2048 + (r & 7) * 256 + ((r >> 3) & 1) * 128 + ((c ^ (r & 7)) << 4);
}
// Row and logical chunk that lane l of 1-KB DMA block q writes.
__device__ __forceinline__ void dma_slot(int q, int l, int* r, int* c) {
  const int half = (l >> 3) & 1;
  *r = (q >> 1) * 16 + (q & 1) * 4 + (l >> 4) + 8 * half;
  *c = (l & 7) ^ (*r & 7);
}

template <int TM, int TN, bool kGateUp, bool kYF32, bool kMX>
__global__ void __launch_bounds__(256, 1) k_tiled(FfnArgs a, int nb_per_tile) {
  constexpr int BM = 32 * TM, BN = 32 * TN;
  constexpr int STAGE = (BM + BN) * 128;
  constexpr int CA = BM / 32, CB = BN / 32;  // 16-B chunks per thread per K block
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  // Tile-major order: the nb_per_tile weight blocks of a row tile are consecutive
  // workgroups, so they read the tile's activation rows at about the same time.
  const int tile_id = blockIdx.x / nb_per_tile;
  if (tile_id >= *a.ntiles) return;
  const int nb = blockIdx.x - tile_id * nb_per_tile;
  const Tile tl = a.tiles[tile_id];
  const int bank = tl.group < a.E ? 0 : 1;
  const int64_t ge = tl.group < a.E ? tl.group : 0;
  const int I = a.bank[bank].I;
  const int H = a.H;
  const int K = kGateUp ? H : I;
  const int fpb = kGateUp ? BN / 2 : BN;  // output features per tile
  const int f0 = nb * fpb;
  if (f0 >= (kGateUp ? I : H)) return;
  const int wrows = kGateUp ? 2 * I : H;  // rows of this expert's weight matrix
  // weights: bf16 rows of K elements, or MXFP4 rows of K/2 bytes with K/32 scale bytes
  const char* wbase;
  const uint8_t* sbase = nullptr;
  if (kMX) {
    wbase = reinterpret_cast<const char*>(kGateUp ? a.bank[bank].w13 : a.bank[bank].w2) +
            ge * (int64_t)wrows * (K / 2);
    sbase = reinterpret_cast<const uint8_t*>(kGateUp ? a.bank[bank].w13_scale : a.bank[bank].w2_scale) +
            ge * (int64_t)wrows * (K / 32);
  } else {
    wbase = reinterpret_cast<const char*>(kGateUp ? a.bank[bank].w13 : a.bank[bank].w2) +
            ge * (int64_t)wrows * K * 2;
  }
  const char* ag[CA];
  const char* bg[CB];
  const uint8_t* bs[CB];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int c = tid + 256 * i;
    const int r = c >> 3, col = (c & 7) * 16;
    const int grow = tl.row0 + (r < tl.nrows ? r : tl.nrows - 1);
    if (kGateUp) {
      const int64_t src = a.a_rowmap ? a.a_rowmap[grow] : grow;
      ag[i] = reinterpret_cast<const char*>(a.a) + src * (int64_t)H * 2 + col;
    } else {
      ag[i] = reinterpret_cast<const char*>(a.h) + (int64_t)grow * a.I_max * 2 + col;
    }
  }
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int c = tid + 256 * i;
    const int r = c >> 3, colc = c & 7;
    int wrow;
    if (kGateUp) {
      const int half = r / (BN / 2), jj = r % (BN / 2), nt = jj >> 4, within = jj & 15;
      const int feat = f0 + half * (BN / 4) + (nt >> 1) * 16 + within;
      wrow = (nt & 1) ? I + feat : feat;
    } else {
      wrow = f0 + r;
    }
    if (kMX) {
      bg[i] = wbase + (int64_t)wrow * (K / 2) + colc * 4;
      bs[i] = sbase + (int64_t)wrow * (K / 32) + (colc >> 2);
    } else {
      bg[i] = wbase + (int64_t)wrow * K * 2 + colc * 16;
      bs[i] = nullptr;
    }
  }
  const int wm = wave & 1, wn = wave >> 1;
  const int m16 = l & 15, g = l >> 4;
  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
  u32x4 ra[CA];
  u32x4 rb[kMX ? 1 : CB];
  uint32_t rq[kMX ? CB : 1], rsc[kMX ? CB : 1];
  auto load_block = [&](int kt) {
    const int64_t o = (int64_t)kt * kTBK * 2;
#pragma unroll
    for (int i = 0; i < CA; ++i) ra[i] = *reinterpret_cast<const u32x4*>(ag[i] + o);
    if (kMX) {
#pragma unroll
      for (int i = 0; i < CB; ++i) {
        rq[i] = *reinterpret_cast<const uint32_t*>(bg[i] + (int64_t)kt * (kTBK / 2));
        rsc[i] = bs[i][kt * (kTBK / 32)];
      }
    } else {
#pragma unroll
      for (int i = 0; i < CB; ++i) rb[kMX ? 0 : i] = *reinterpret_cast<const u32x4*>(bg[i] + o);
    }
  };
  auto store_block = [&](char* st) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int c = tid + 256 * i;
      *reinterpret_cast<u32x4*>(st + lds_off(c >> 3, c & 7)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int c = tid + 256 * i;
      char* dst = st + BM * 128 + lds_off(c >> 3, c & 7);
      if (kMX) {
        const float sc = e8m0_f32(rsc[i]);
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(rq[i], sc, 0);
        bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(rq[i], sc, 1);
        bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(rq[i], sc, 2);
        bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(rq[i], sc, 3);
        u32x4 v;
        v[0] = __builtin_bit_cast(uint32_t, p0);
        v[1] = __builtin_bit_cast(uint32_t, p1);
        v[2] = __builtin_bit_cast(uint32_t, p2);
        v[3] = __builtin_bit_cast(uint32_t, p3);
        *reinterpret_cast<u32x4*>(dst) = v;
      } else {
        *reinterpret_cast<u32x4*>(dst) = rb[kMX ? 0 : i];
      }
    }
  };
  load_block(0);
  store_block(smem);
  __syncthreads();
  const int KT = K / kTBK;
  for (int kt = 0; kt < KT; ++kt) {
    const char* cur = smem + (kt & 1) * STAGE;
    if (kt + 1 < KT) load_block(kt + 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 fa[TM], fb[TN];
      const int kb = g * 32 + ks * 16;
#pragma unroll
      for (int t = 0; t < TM; ++t)
        fa[t] = *reinterpret_cast<const bf16x8*>(cur + lds_off(wm * (BM / 2) + t * 16 + m16, kb >> 4));
#pragma unroll
      for (int t = 0; t < TN; ++t)
        fb[t] = *reinterpret_cast<const bf16x8*>(cur + BM * 128 +
                                                 lds_off(wn * (BN / 2) + t * 16 + m16, kb >> 4));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) store_block(smem + ((kt + 1) & 1) * STAGE);
    __syncthreads();
  }
  // epilogue: lane holds D[row 4g+i][column m16] of each 16 x 16 sub-tile
#pragma unroll
  for (int mt = 0; mt < TM; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rl = wm * (BM / 2) + mt * 16 + 4 * g + i;
      if (rl >= tl.nrows) continue;
      const int64_t row = tl.row0 + rl;
      if (kGateUp) {
#pragma unroll
        for (int p = 0; p < TN / 2; ++p) {
          const int feat = f0 + wn * (BN / 4) + p * 16 + m16;
          const float hv = silu_mul(acc[mt][2 * p][i], acc[mt][2 * p + 1][i]);
          reinterpret_cast<uint16_t*>(a.h)[row * a.I_max + feat] = f32_to_bf16(hv);
        }
      } else {
#pragma unroll
        for (int nt = 0; nt < TN; ++nt) {
          const int64_t o = row * H + f0 + wn * (BN / 2) + nt * 16 + m16;
          if (kYF32) reinterpret_cast<float*>(a.y)[o] = acc[mt][nt][i];
          else reinterpret_cast<uint16_t*>(a.y)[o] = f32_to_bf16(acc[mt][nt][i]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// Tiled kernel, DMA version (bf16 weights): the same tile arithmetic as k_tiled, but the
// K blocks go from global memory straight into LDS with global_load_lds_dwordx4 (no
// register staging), through an S-stage ring so that each load has S-1 K blocks of MFMA
// work to hide behind. LDS layout of a K block (128 B per row): each 16-row group takes
// 2 KB = eight 256-B lines; line j holds row j in its low 128 B and row 8 + j in its high
// 128 B, and the 16-B chunk c of row r sits at chunk c ^ (r & 7). Measured on MI355X, this
// lets the fragment reads of 16 consecutive rows at one chunk run at the full LDS rate
// (~250 B/clk/CU) where padded or plainly swizzled rows reach half of it. A wavefront's
// DMA writes 1 KB contiguously (16 B per lane, lane order), i.e. 4 + 4 rows of a group,
// and each lane's global address absorbs the layout.
#ifndef MOE_T2_TM
#define MOE_T2_TM 4
#endif
#ifndef MOE_T2_TN
#define MOE_T2_TN 4
#endif
#ifndef MOE_T2_WGM
#define MOE_T2_WGM 2
#endif
#ifndef MOE_T2_WGN
#define MOE_T2_WGN 2
#endif
#ifndef MOE_T2_STAGES
#define MOE_T2_STAGES 2
#endif
#ifndef MOE_T2_MX_STAGES
#define MOE_T2_MX_STAGES 3
#endif
#ifndef MOE_T2_WAVES_PER_SIMD
#define MOE_T2_WAVES_PER_SIMD 2
#endif
constexpr int kT2Threads = 64 * MOE_T2_WGM * MOE_T2_WGN;
constexpr int kT2M = MOE_T2_WGM * 16 * MOE_T2_TM, kT2N = MOE_T2_WGN * 16 * MOE_T2_TN;
static_assert(kT2M == kTBM, "the MXFP4 tile list serves both tiled kernels");

typedef __attribute__((address_space(3))) void lds_void;

// 16 B per lane from global memory into LDS at lds + 16 * lane (a device-only wrapper: the
// target builtin must not appear in code the host pass instantiates).
__device__ __forceinline__ void dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, 0);
}
// 4 B per lane from global memory into LDS at lds + 4 * lane (device-only wrapper).
__device__ __forceinline__ void dma4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 4, 0, 0);
}

// Eight E2M1 values (one 32-bit word, low nibble first) times their E8M0 block scale, as
// the bf16 fragment of one MFMA k-step (v_cvt_scalef32_pk_bf16_fp4 is exact: every
// E2M1 value times a power of two in range is a bf16).
__device__ __forceinline__ bf16x8 e2m1x8_bf16(uint32_t w, float scale) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup of WGM x WGN wavefronts; each wavefront computes (16 TM) x (16 TN).
// kMX: MXFP4 weights. A K block of a weight row is then 32 B of E2M1 codes plus 2 E8M0
// scale bytes; the ring stages the codes (32 B a row: the 8-B quarter u of row r at
// quarter u ^ 2 ((r >> 3) & 1), which spreads the 64-bit fragment reads of 16 rows over
// all banks) and 4 scale bytes a row (those of K blocks kt & ~1 and (kt & ~1) + 1, one
// aligned dword), and fragments are decoded to bf16 in registers as they are read.
template <int TM, int TN, int WGM, int WGN, int S, bool kGateUp, bool kYF32, bool kMX>
__global__ void __launch_bounds__(64 * WGM * WGN, MOE_T2_WAVES_PER_SIMD) k_tiled2(FfnArgs a, int nb_per_tile) {
  constexpr int NW = WGM * WGN;
  constexpr int BM = WGM * 16 * TM, BN = WGN * 16 * TN;
  constexpr int BSTAGE = kMX ? BN * 32 + BN * 4 : BN * 128;  // weight bytes of a stage
  constexpr int STAGE = BM * 128 + BSTAGE;
  constexpr int RPI = NW * 8;                  // LDS rows filled per DMA instruction round
  constexpr int CA = BM / RPI;                 // DMA instructions per thread per K block: A,
  constexpr int CB = kMX ? BN * 32 / (1024 * NW) : BN / RPI;  // B,
  constexpr int CS = kMX ? 1 : 0;                              // MXFP4 scales
  constexpr int OPS = CA + CB + CS;
  static_assert(BM % RPI == 0 && BN % RPI == 0 && BM % 16 == 0, "tile rows per DMA round");
  static_assert(!kMX || (BN * 32 % (1024 * NW) == 0 && BN == 32 * NW), "MXFP4 DMA rounds");
  __shared__ __attribute__((aligned(1024))) char smem[S * STAGE];
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  // tile-major order, as in k_tiled
  const int tidx = blockIdx.x / nb_per_tile;
  if (tidx >= *a.ntiles) return;
  const int nb = blockIdx.x - tidx * nb_per_tile;
  const Tile tl = a.tiles[tidx];
  const int bank = tl.group < a.E ? 0 : 1;
  const int64_t ge = tl.group < a.E ? tl.group : 0;
  const int I = a.bank[bank].I;
  const int H = a.H;
  const int K = kGateUp ? H : I;
  const int fpb = kGateUp ? BN / 2 : BN;
  const int f0 = nb * fpb;
  if (f0 >= (kGateUp ? I : H)) return;
  const int64_t wrows = kGateUp ? 2 * I : H;  // rows of this expert's weight matrix
  const int64_t wrow_bytes = kMX ? K / 2 : K * 2;
  const char* wbase = reinterpret_cast<const char*>(kGateUp ? a.bank[bank].w13 : a.bank[bank].w2) +
                      ge * wrows * wrow_bytes;
  // weight row of B-tile row r (gate/up: each N-wavefront block of 16 TN rows holds the
  // gate and up rows of 8 TN features, alternating by 16)
  auto weight_row = [&](int r) {
    if (kGateUp) {
      const int blk = r / (16 * TN), jj = r % (16 * TN), nt = jj >> 4, within = jj & 15;
      const int feat = f0 + blk * (8 * TN) + (nt >> 1) * 16 + within;
      return (nt & 1) ? I + feat : feat;
    }
    return f0 + r;
  };
  // DMA instruction i of wavefront w fills 1-KB block q = NW i + w of the A (then B) tile
  const char* ag[CA];
  const char* bg[CB];
  const uint8_t* sg = nullptr;
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    int r, cc;
    dma_slot(NW * i + wave, l, &r, &cc);
    const int col = cc * 16;
    const int grow = tl.row0 + (r < tl.nrows ? r : tl.nrows - 1);
    if (kGateUp) {
      const int64_t src = a.a_rowmap ? a.a_rowmap[grow] : grow;
      ag[i] = reinterpret_cast<const char*>(a.a) + src * (int64_t)H * 2 + col;
    } else {
      ag[i] = reinterpret_cast<const char*>(a.h) + (int64_t)grow * a.I_max * 2 + col;
    }
  }
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    if (kMX) {
      // lane l: row 32 q + l / 2, physical 16-B half l % 2 of its 32-B slice
      const int r = 32 * (NW * i + wave) + (l >> 1);
      const int lh = (l & 1) ^ ((r >> 3) & 1);
      bg[i] = wbase + weight_row(r) * wrow_bytes + lh * 16;
    } else {
      int r, cc;
      dma_slot(NW * i + wave, l, &r, &cc);
      bg[i] = wbase + weight_row(r) * wrow_bytes + cc * 16;
    }
  }
  if (kMX) {
    // lanes 0..31 of wavefront w fetch the scale dword of B-tile row 32 w + lane
    const uint8_t* sbase = reinterpret_cast<const uint8_t*>(kGateUp ? a.bank[bank].w13_scale
                                                                    : a.bank[bank].w2_scale) +
                           ge * wrows * (K / 32);
    sg = sbase + weight_row(32 * wave + (l & 31)) * (int64_t)(K / 32);
  }
  auto issue = [&](int kt, int stage) {
    const int64_t o = (int64_t)kt * 128;
    char* st = smem + stage * STAGE;
#pragma unroll
    for (int i = 0; i < CA; ++i) dma16(ag[i] + o, st + (NW * i + wave) * 1024);
    if (kMX) {
#pragma unroll
      for (int i = 0; i < CB; ++i) dma16(bg[i] + (int64_t)kt * 32, st + BM * 128 + (NW * i + wave) * 1024);
      if (l < 32) dma4(sg + (kt & ~1) * 2, st + BM * 128 + BN * 32 + wave * 128);
    } else {
#pragma unroll
      for (int i = 0; i < CB; ++i) dma16(bg[i] + o, st + BM * 128 + (NW * i + wave) * 1024);
    }
  };
  const int wm = wave % WGM, wn = wave / WGM;
  const int m16 = l & 15, g = l >> 4;
  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
  const int KT = K / kTBK;
  int arow[TM], brow[TN];
#pragma unroll
  for (int t = 0; t < TM; ++t) arow[t] = wm * (16 * TM) + t * 16 + m16;
#pragma unroll
  for (int t = 0; t < TN; ++t) brow[t] = wn * (16 * TN) + t * 16 + m16;
#pragma unroll
  for (int p = 0; p < S - 1; ++p)
    if (p < KT) issue(p, p);
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + S - 2 < KT) wait_vmcnt<(S - 2) * OPS>();
    else wait_vmcnt<0>();
    // A plain barrier, not __syncthreads(): its fence would wait for every outstanding
    // DMA of the ring. The wait above already covers this thread's part of block kt.
    __builtin_amdgcn_s_barrier();
    if (kt + S - 1 < KT) issue(kt + S - 1, (kt + S - 1) % S);
    const char* cur = smem + (kt % S) * STAGE;
    // MXFP4: this lane's 16 codes (elements 16 g .. 16 g + 15 of the K block) and scale
    uint2 wq[kMX ? TN : 1];
    float wsc[kMX ? TN : 1];
    if (kMX) {
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const char* rb = cur + BM * 128 + brow[t] * 32;
        // two 32-bit reads: with one 64-bit read the compiler makes it wait for all DMA
        const char* q = rb + 8 * (g ^ (((brow[t] >> 3) & 1) << 1));
        wq[t].x = *reinterpret_cast<const uint32_t*>(q);
        wq[t].y = *reinterpret_cast<const uint32_t*>(q + 4);
        wsc[t] = e8m0_f32(*reinterpret_cast<const uint8_t*>(cur + BM * 128 + BN * 32 + 4 * brow[t] +
                                                             (kt & 1) * 2 + (g >> 1)));
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 fa[TM], fb[TN];
      const int c = 2 * g + ks;  // logical 16-B chunk
#pragma unroll
      for (int t = 0; t < TM; ++t)
        fa[t] = *reinterpret_cast<const bf16x8*>(cur + lds_off(arow[t], c));
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        if (kMX) fb[t] = e2m1x8_bf16(ks ? wq[t].y : wq[t].x, wsc[t]);
        else fb[t] = *reinterpret_cast<const bf16x8*>(cur + BM * 128 + lds_off(brow[t], c));
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int mt = 0; mt < TM; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rl = wm * (16 * TM) + mt * 16 + 4 * g + i;
      if (rl >= tl.nrows) continue;
      const int64_t row = tl.row0 + rl;
      if (kGateUp) {
#pragma unroll
        for (int p = 0; p < TN / 2; ++p) {
          const int feat = f0 + wn * (8 * TN) + p * 16 + m16;
          const float hv = silu_mul(acc[mt][2 * p][i], acc[mt][2 * p + 1][i]);
          reinterpret_cast<uint16_t*>(a.h)[row * a.I_max + feat] = f32_to_bf16(hv);
        }
      } else {
#pragma unroll
        for (int nt = 0; nt < TN; ++nt) {
          const int64_t o = row * H + f0 + wn * (16 * TN) + nt * 16 + m16;
          if (kYF32) reinterpret_cast<float*>(a.y)[o] = acc[mt][nt][i];
          else reinterpret_cast<uint16_t*>(a.y)[o] = f32_to_bf16(acc[mt][nt][i]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// fp8 path (E4M3 weights with fp32 128 x 128 block scales, activations E4M3 with fp32
// 1 x 128 scales), the FP8 grouped GEMM with fused SwiGLU and re-quantisation of GC-MoE
// (key_changes, fourth item) re-planned for gfx950:
//  - v_mfma_scale_f32_16x16x128_f8f6f4 with unit E8M0 scales computes one 128-wide K block
//    of a 16 x 16 tile exactly; the fp32 block scales (not powers of two, so not foldable
//    into the MFMA's own scale operands) are applied per K block on the VALU:
//    acc += partial * (s_w * s_x[token]).
//  - weights are the MFMA A operand, read straight from HBM into registers (32 B/lane,
//    one 128-B K block of 16 rows per wavefront and matrix, prefetched one block ahead);
//    the tile's <= 128 activation rows and their scales are staged in LDS once per K
//    block and shared by the 8 wavefronts of the workgroup (128 output features).
//  - gate/up epilogue: h = SiLU(g) * u in fp32, per-token amax over the workgroup's 128
//    features (wavefront shuffles, then LDS across wavefronts), scale = amax / 448,
//    E4M3 codes of h / scale -- exactly one 1 x 128 quantisation block per workgroup.
#ifndef MOE_F8_STAGES_GU
#define MOE_F8_STAGES_GU 3
#endif
#ifndef MOE_F8_STAGES_DN
#define MOE_F8_STAGES_DN 4
#endif
constexpr int kF8TileM = 128;
constexpr int kF8Feat = 128;
constexpr int kF8K = 128;

// fp32 -> E4M3FN code, round to nearest even, saturating at +-448 (NaN -> 0x7F).
// Written from the format: magnitudes below 2^-6 lie on the subnormal grid m * 2^-9;
// above, a value 2^e * (1 + f) keeps 3 fraction bits.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  if (!(a == a)) return 0x7Fu;
  if (a >= 464.0f) return sign | 0x7Eu;
  const int ex = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;
  if (ex < -6) return sign | (uint32_t)__builtin_rintf(a * 512.0f);      // 0..8
  float m = __builtin_rintf(__uint_as_float((uint32_t)(127 + 3 - ex) << 23) * a);  // 8..16
  int e = ex;
  if (m == 16.0f) { m = 8.0f; ++e; }
  uint32_t code = ((uint32_t)(e + 7) << 3) | ((uint32_t)m - 8u);
  return sign | (code > 0x7Eu ? 0x7Eu : code);
}

__device__ __forceinline__ float wave_max16(float v) {  // max over lanes with equal l % 16
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}

// Quantise rows of a bf16 [n, H] matrix: one workgroup per row, 16 lanes per 1 x 128 block.
__global__ void __launch_bounds__(256) k_quant_rows_fp8(const uint16_t* __restrict__ x, int H,
                                                        uint8_t* __restrict__ q,
                                                        float* __restrict__ qs) {
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x;
  const int nblk = H / 128;
  for (int b0 = 0; b0 < nblk; b0 += 16) {
    const int b = b0 + (t >> 4);
    const int j = t & 15;
    float v[8];
    float am = 0.0f;
    if (b < nblk) {
      uint4 w = *reinterpret_cast<const uint4*>(x + row * H + b * 128 + j * 8);
      v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
      v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
#pragma unroll
      for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[i]));
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, 16));
    if (b < nblk) {
      const float sc = am == 0.0f ? 1.0f : __fdiv_rn(am, 448.0f);
      uint2 c;
      c.x = e4m3_code(__fdiv_rn(v[0], sc)) | (e4m3_code(__fdiv_rn(v[1], sc)) << 8) |
            (e4m3_code(__fdiv_rn(v[2], sc)) << 16) | (e4m3_code(__fdiv_rn(v[3], sc)) << 24);
      c.y = e4m3_code(__fdiv_rn(v[4], sc)) | (e4m3_code(__fdiv_rn(v[5], sc)) << 8) |
            (e4m3_code(__fdiv_rn(v[6], sc)) << 16) | (e4m3_code(__fdiv_rn(v[7], sc)) << 24);
      *reinterpret_cast<uint2*>(q + row * H + b * 128 + j * 8) = c;
      if (j == 0) qs[row * nblk + b] = sc;
    }
  }
}

__device__ __forceinline__ i32x8 ld32(const void* p) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
  u32x4 a = q[0], b = q[1];
  i32x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

template <bool kGateUp>
__global__ void __launch_bounds__(512, 2) k_fp8(FfnArgs a, int fb_per_tile) {
  // Each K block of the workgroup's operands -- its 128 (down) or 256 (gate/up) weight
  // rows, the tile's 128 activation rows (both in the full-rate layout of lds_off) and the
  // fp32 scales of both -- goes global -> LDS by DMA through an S-stage ring, requested
  // S-1 blocks ahead. The K loop issues no other vector-memory load and reads no other LDS
  // object, so its only vector-memory wait is the one for the oldest stage.
  constexpr int S = kGateUp ? MOE_F8_STAGES_GU : MOE_F8_STAGES_DN;
  constexpr int WR = kGateUp ? 2 * kF8Feat : kF8Feat;   // weight rows per stage
  constexpr int WB = WR * 128;                           // weight bytes per stage
  constexpr int ACT = kF8TileM * 128;
  constexpr int SCL = 8 * 128;  // per wavefront: its 16 rows' scales, then the weight scales
  constexpr int STG = WB + ACT + SCL;
  constexpr int NWD = WR / 64;                           // weight DMA ops per thread
  constexpr int A = NWD + 2 + 1;                         // DMA ops per thread per K block
  // The ring is the kernel's only LDS object (the epilogue's amax table reuses it): with
  // a second one the compiler tags LDS accesses with alias scopes and then makes every
  // ring read wait for all outstanding DMA, not just for the oldest stage's.
  __shared__ __attribute__((aligned(1024))) char ring[S * STG];
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int m16 = l & 15, g = l >> 4;
  const int tile_id = blockIdx.x / fb_per_tile;
  const int fb = blockIdx.x - tile_id * fb_per_tile;
  if (tile_id >= *a.ntiles) return;
  const Tile tl = a.tiles[tile_id];
  const int bank = tl.group < a.E ? 0 : 1;
  const int64_t ge = tl.group < a.E ? tl.group : 0;
  const int I = a.bank[bank].I;
  const int H = a.H;
  const int K = kGateUp ? H : I;
  const int f0 = fb * kF8Feat;
  if (f0 >= (kGateUp ? I : H)) return;
  const int KB = K / kF8K;
  const int ntb = (tl.nrows + 15) >> 4;
  // weight DMA sources: block q = 8 i + wave of the weight area; tile rows r < 128 are the
  // gate (or down) rows f0 + r, rows 128.. the up rows I + f0 + r - 128
  const uint8_t* wbase = reinterpret_cast<const uint8_t*>(kGateUp ? a.bank[bank].w13 : a.bank[bank].w2) +
                         ge * (int64_t)(kGateUp ? 2 * I : H) * K;
  const uint8_t* wp[NWD];
#pragma unroll
  for (int i = 0; i < NWD; ++i) {
    int r, c;
    dma_slot(8 * i + wave, l, &r, &c);
    const int wrow = r < kF8Feat ? f0 + r : I + f0 + (r - kF8Feat);
    wp[i] = wbase + (int64_t)wrow * K + c * 16;
  }
  // activation DMA sources: block q = 8 i + wave of the activation area
  const uint8_t* ap[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    int r, c;
    dma_slot(8 * i + wave, l, &r, &c);
    const int grow = tl.row0 + (r < tl.nrows ? r : 0);
    if (kGateUp) {
      const int64_t src = a.a_rowmap ? a.a_rowmap[grow] : grow;
      ap[i] = a.a_q + src * (int64_t)H + c * 16;
    } else {
      ap[i] = reinterpret_cast<const uint8_t*>(a.h) + (int64_t)grow * a.I_max + c * 16;
    }
  }
  // scales: lanes 0..15 of wavefront w fetch those of rows 16 w + lane, lanes 16 and 17
  // the gate (or down) and up weight block scales, into the wavefront's 128-B slot
  const float* sp;
  if (l < 16) {
    const int r = wave * 16 + m16;
    const int grow = tl.row0 + (r < tl.nrows ? r : 0);
    if (kGateUp) {
      const int64_t src = a.a_rowmap ? a.a_rowmap[grow] : grow;
      sp = a.a_qscale + src * (H / kF8K);
    } else {
      sp = a.h_scale + (int64_t)grow * (a.I_max / kF8K);
    }
  } else if (kGateUp) {
    const float* sb = reinterpret_cast<const float*>(a.bank[bank].w13_scale) + ge * (2 * I / 128) * (int64_t)KB;
    sp = sb + (int64_t)((l == 16 ? f0 : I + f0) / 128) * KB;
  } else {
    const float* sb = reinterpret_cast<const float*>(a.bank[bank].w2_scale) + ge * (H / 128) * (int64_t)KB;
    sp = sb + (int64_t)(f0 / 128) * KB;
  }
  auto issue = [&](int kb) {
    char* st = ring + (kb % S) * STG;
    const int64_t o = (int64_t)kb * kF8K;
#pragma unroll
    for (int i = 0; i < NWD; ++i) dma16(wp[i] + o, st + (8 * i + wave) * 1024);
    dma16(ap[0] + o, st + WB + wave * 1024);
    dma16(ap[1] + o, st + WB + (8 + wave) * 1024);
    if (l < (kGateUp ? 18 : 17)) dma4(sp + kb, st + WB + ACT + wave * 128);
  };
  f32x4 acc0[8], acc1[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) { acc0[t] = f32x4{0, 0, 0, 0}; acc1[t] = f32x4{0, 0, 0, 0}; }
#pragma unroll
  for (int p = 0; p < S - 1; ++p)
    if (p < KB) issue(p);
  const int wr0 = wave * 16 + m16;  // this lane's gate (or down) weight row in the tile
  for (int kb = 0; kb < KB; ++kb) {
    // block kb has landed once at most (blocks issued after it) * A ops are outstanding
    if (kb + S - 2 < KB) wait_vmcnt<(S - 2) * A>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (kb + S - 1 < KB) issue(kb + S - 1);
    const char* st = ring + (kb % S) * STG;
    i32x8 wa, wb;
    {
      const u32x4 p0 = *reinterpret_cast<const u32x4*>(st + lds_off(wr0, 2 * g));
      const u32x4 p1 = *reinterpret_cast<const u32x4*>(st + lds_off(wr0, 2 * g + 1));
      wa[0] = p0[0]; wa[1] = p0[1]; wa[2] = p0[2]; wa[3] = p0[3];
      wa[4] = p1[0]; wa[5] = p1[1]; wa[6] = p1[2]; wa[7] = p1[3];
      if (kGateUp) {
        const u32x4 q0 = *reinterpret_cast<const u32x4*>(st + lds_off(kF8Feat + wr0, 2 * g));
        const u32x4 q1 = *reinterpret_cast<const u32x4*>(st + lds_off(kF8Feat + wr0, 2 * g + 1));
        wb[0] = q0[0]; wb[1] = q0[1]; wb[2] = q0[2]; wb[3] = q0[3];
        wb[4] = q1[0]; wb[5] = q1[1]; wb[6] = q1[2]; wb[7] = q1[3];
      } else {
        wb = wa;
      }
    }
    const float sw0 = *reinterpret_cast<const float*>(st + WB + ACT + wave * 128 + 64);
    const float sw1 = kGateUp ? *reinterpret_cast<const float*>(st + WB + ACT + wave * 128 + 68) : 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (t < ntb) {
        const int r = t * 16 + m16;
        const u32x4 x0 = *reinterpret_cast<const u32x4*>(st + WB + lds_off(r, 2 * g));
        const u32x4 x1 = *reinterpret_cast<const u32x4*>(st + WB + lds_off(r, 2 * g + 1));
        i32x8 xb;
        xb[0] = x0[0]; xb[1] = x0[1]; xb[2] = x0[2]; xb[3] = x0[3];
        xb[4] = x1[0]; xb[5] = x1[1]; xb[6] = x1[2]; xb[7] = x1[3];
        const float sx = *reinterpret_cast<const float*>(st + WB + ACT + t * 128 + m16 * 4);
        const f32x4 z = {0, 0, 0, 0};
        f32x4 p0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wa, xb, z, 0, 0, 0, 127, 0, 127);
        const float c0 = sw0 * sx;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc0[t][i] += p0[i] * c0;
        if (kGateUp) {
          f32x4 p1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wb, xb, z, 0, 0, 0, 127, 0, 127);
          const float c1 = sw1 * sx;
#pragma unroll
          for (int i = 0; i < 4; ++i) acc1[t][i] += p1[i] * c1;
        }
      }
    }
  }
  __syncthreads();
  float(*red)[kF8TileM] = reinterpret_cast<float(*)[kF8TileM]>(ring);  // [8][128] amax table
  const int fw = f0 + wave * 16;
  // lane holds D[feature fw + 4g + i][token t*16 + m16]
  if (kGateUp) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      float am = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc0[t][i] = silu_mul(acc0[t][i], acc1[t][i]);
        am = fmaxf(am, fabsf(acc0[t][i]));
      }
      am = wave_max16(am);
      if (g == 0) red[wave][t * 16 + m16] = am;
    }
    __syncthreads();
    uint8_t* hq = reinterpret_cast<uint8_t*>(a.h);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int tok = t * 16 + m16;
      if (tok >= tl.nrows) continue;
      float am = 0.0f;
#pragma unroll
      for (int w = 0; w < 8; ++w) am = fmaxf(am, red[w][tok]);
      const float sc = am == 0.0f ? 1.0f : __fdiv_rn(am, 448.0f);
      uint32_t c = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) c |= e4m3_code(__fdiv_rn(acc0[t][i], sc)) << (8 * i);
      const int64_t row = tl.row0 + tok;
      *reinterpret_cast<uint32_t*>(hq + row * a.I_max + fw + 4 * g) = c;
      if (wave == 0 && g == 0) a.h_scale[row * (a.I_max / kF8K) + f0 / kF8K] = sc;
    }
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int tok = t * 16 + m16;
      if (tok >= tl.nrows) continue;
      const int64_t o = (int64_t)(tl.row0 + tok) * H + fw + 4 * g;
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.y) + o) =
          make_float4(acc0[t][0], acc0[t][1], acc0[t][2], acc0[t][3]);
    }
  }
}

}  // namespace

bool ffn_shape_ok(moe_dtype wdt, int32_t H, int32_t I) {
  switch (wdt) {
    case MOE_F32:
    case MOE_BF16: return H % 64 == 0 && I % 64 == 0;
    case MOE_FP8_E4M3: return H % kF8Feat == 0 && I % kF8Feat == 0;
    case MOE_MXFP4: return H % kTBN == 0 && I % (kTBN / 2) == 0 && H % kTBK == 0 && I % kTBK == 0;
  }
  return false;
}

int32_t ffn_tile_m(moe_dtype wdt, int32_t rows, int32_t groups, int32_t H, int32_t I_routed,
                   int32_t I_shared) {
  if (wdt == MOE_FP8_E4M3) return kF8TileM;
  // Few rows per expert: stream the weights (each weight element read once per tile of
  // <= 16 rows). Many rows: LDS-tiled GEMM with 128-row tiles.
  if (wdt == MOE_MXFP4) return kTBM;
  const bool t2_ok = H % kT2N == 0 && I_routed % (kT2N / 2) == 0 && I_shared % (kT2N / 2) == 0;
  if (wdt == MOE_BF16 && t2_ok && (int64_t)rows > 32 * (int64_t)groups) return kT2M;
  return kStreamTileM;
}

size_t ffn_scratch_bytes(moe_dtype wdt, int32_t rows_total, int32_t H, int32_t I_max) {
  (void)H;
  if (wdt == MOE_FP8_E4M3) {
    const size_t q = ((size_t)rows_total * I_max + 255) / 256 * 256;
    return q + ((size_t)rows_total * (I_max / kF8K) * sizeof(float) + 255) / 256 * 256;
  }
  const size_t hb = (wdt == MOE_F32) ? 4 : 2;
  return ((size_t)rows_total * I_max * hb + 255) / 256 * 256;
}

hipError_t launch_grouped_ffn(FfnArgs a, void* scratch, hipStream_t s, hipEvent_t mid_event) {
  if (a.max_tiles <= 0) {
    return mid_event ? hipEventRecord(mid_event, s) : hipSuccess;
  }
  a.h = scratch;
  if (a.wdt == MOE_FP8_E4M3) {
    a.h_scale = reinterpret_cast<float*>(reinterpret_cast<char*>(scratch) +
                                         ((size_t)a.rows_total * a.I_max + 255) / 256 * 256);
    const int nb_gu = a.I_max / kF8Feat, nb_dn = a.H / kF8Feat;
    hipLaunchKernelGGL(k_fp8<true>, dim3(a.max_tiles * nb_gu), dim3(512), 0, s, a, nb_gu);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (mid_event && (err = hipEventRecord(mid_event, s)) != hipSuccess) return err;
    hipLaunchKernelGGL(k_fp8<false>, dim3(a.max_tiles * nb_dn), dim3(512), 0, s, a, nb_dn);
    return hipGetLastError();
  }
  const int fb_gu = (a.I_max + kFeatPerWG - 1) / kFeatPerWG;
  const int fb_dn = (a.H + kFeatPerWG - 1) / kFeatPerWG;
  const bool f32 = a.wdt == MOE_F32;
  const bool yf32 = a.y_dt == MOE_F32;
  dim3 blk(256);
  if (a.tile_m == kT2M && a.wdt == MOE_BF16) {
    const int nb_gu = a.I_max / (kT2N / 2), nb_dn = a.H / kT2N;
    hipLaunchKernelGGL((k_tiled2<MOE_T2_TM, MOE_T2_TN, MOE_T2_WGM, MOE_T2_WGN, MOE_T2_STAGES, true, false, false>), dim3(a.max_tiles * nb_gu), dim3(kT2Threads), 0, s, a, nb_gu);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (mid_event && (err = hipEventRecord(mid_event, s)) != hipSuccess) return err;
    if (yf32)
      hipLaunchKernelGGL((k_tiled2<MOE_T2_TM, MOE_T2_TN, MOE_T2_WGM, MOE_T2_WGN, MOE_T2_STAGES, false, true, false>), dim3(a.max_tiles * nb_dn), dim3(kT2Threads), 0, s, a, nb_dn);
    else
      hipLaunchKernelGGL((k_tiled2<MOE_T2_TM, MOE_T2_TN, MOE_T2_WGM, MOE_T2_WGN, MOE_T2_STAGES, false, false, false>), dim3(a.max_tiles * nb_dn), dim3(kT2Threads), 0, s, a, nb_dn);
    return hipGetLastError();
  }
  // MXFP4 through the DMA kernel when every weight row's scale bytes are dword aligned
  // (K % 128 for both products)
  if (a.tile_m == kT2M && a.wdt == MOE_MXFP4 && a.H % kT2N == 0 && a.bank[0].I % 128 == 0 &&
      (!a.has_shared || a.bank[1].I % 128 == 0)) {
    const int nb_gu = a.I_max / (kT2N / 2), nb_dn = a.H / kT2N;
    hipLaunchKernelGGL((k_tiled2<MOE_T2_TM, MOE_T2_TN, MOE_T2_WGM, MOE_T2_WGN, MOE_T2_MX_STAGES, true, false, true>), dim3(a.max_tiles * nb_gu), dim3(kT2Threads), 0, s, a, nb_gu);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (mid_event && (err = hipEventRecord(mid_event, s)) != hipSuccess) return err;
    if (yf32)
      hipLaunchKernelGGL((k_tiled2<MOE_T2_TM, MOE_T2_TN, MOE_T2_WGM, MOE_T2_WGN, MOE_T2_MX_STAGES, false, true, true>), dim3(a.max_tiles * nb_dn), dim3(kT2Threads), 0, s, a, nb_dn);
    else
      hipLaunchKernelGGL((k_tiled2<MOE_T2_TM, MOE_T2_TN, MOE_T2_WGM, MOE_T2_WGN, MOE_T2_MX_STAGES, false, false, true>), dim3(a.max_tiles * nb_dn), dim3(kT2Threads), 0, s, a, nb_dn);
    return hipGetLastError();
  }
  if (a.tile_m == kTBM) {
    const int nb_gu = a.I_max / (kTBN / 2), nb_dn = a.H / kTBN;
    const bool mx = a.wdt == MOE_MXFP4;
    if (mx)
      hipLaunchKernelGGL((k_tiled<kTTM, kTTN, true, false, true>), dim3(a.max_tiles * nb_gu), blk, 0, s, a, nb_gu);
    else
      hipLaunchKernelGGL((k_tiled<kTTM, kTTN, true, false, false>), dim3(a.max_tiles * nb_gu), blk, 0, s, a, nb_gu);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (mid_event && (err = hipEventRecord(mid_event, s)) != hipSuccess) return err;
    if (mx && yf32)
      hipLaunchKernelGGL((k_tiled<kTTM, kTTN, false, true, true>), dim3(a.max_tiles * nb_dn), blk, 0, s, a, nb_dn);
    else if (mx)
      hipLaunchKernelGGL((k_tiled<kTTM, kTTN, false, false, true>), dim3(a.max_tiles * nb_dn), blk, 0, s, a, nb_dn);
    else if (yf32)
      hipLaunchKernelGGL((k_tiled<kTTM, kTTN, false, true, false>), dim3(a.max_tiles * nb_dn), blk, 0, s, a, nb_dn);
    else
      hipLaunchKernelGGL((k_tiled<kTTM, kTTN, false, false, false>), dim3(a.max_tiles * nb_dn), blk, 0, s, a, nb_dn);
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

hipError_t launch_quant_rows_fp8(const void* x, int32_t n, int32_t H, uint8_t* q, float* qs,
                                 hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_quant_rows_fp8, dim3(n), dim3(256), 0, s,
                     reinterpret_cast<const uint16_t*>(x), H, q, qs);
  return hipGetLastError();
}

}  // namespace moe
