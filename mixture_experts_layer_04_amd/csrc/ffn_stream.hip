// Streaming grouped-FFN kernels (few rows per expert, e.g. decode), which are bound by
// streaming the weights of the touched experts ("GC-MoE: Overlapping Expert-Parallel
// Token Dispatch with FP8/FP4 Grouped GEMM via CUDA Green Contexts", why_it_matters).
// The weights are the MFMA A operand (16 output features per wavefront), the <= 16 rows
// of the tile the B operand. Each lane loads 32 contiguous bytes of its weight row per
// step (a full 128-B line per 4 lanes) straight from HBM into registers: a weight element
// is read exactly once per tile and never staged in LDS. bf16 uses
// v_mfma_f32_16x16x32_bf16, fp32 v_mfma_f32_16x16x4_f32. Because a dot product may be
// summed in any order, the K index carried by lane group kq and register slot j is
// k0 + 16*kq + j (bf16) -- the same map for A and B -- which makes every load contiguous.
#include "ffn_common.h"

namespace moe {
namespace {

constexpr int kFeatPerWG = 64;  // 4 wavefronts x 16 output features

struct Frag32 {  // 32 bytes per lane
  u32x4 lo, hi;
};

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

// K steps per loop iteration of the streaming kernels (tuning constants).
#ifndef MOE_STREAM_UNROLL_GU
#define MOE_STREAM_UNROLL_GU 2
#endif
#ifndef MOE_STREAM_ROWS_GU  // 16-row weight groups per wavefront (bf16)
#define MOE_STREAM_ROWS_GU 4
#endif
#ifndef MOE_STREAM_ROWS_DN
#define MOE_STREAM_ROWS_DN 1
#endif
#ifndef MOE_STREAM_UNROLL_DN
#define MOE_STREAM_UNROLL_DN 8
#endif
// Weight fragment: ordinary cached loads (on MI355X they measured faster than
// non-temporal ones for this many-rows-at-once pattern).
__device__ __forceinline__ Frag32 load_w(const void* p) { return load_c(p); }
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

// Gate/up + SwiGLU. Workgroup = (tile, block of 64 R h features); wavefront w computes
// features [f0, f0 + 16 R) of h: gate rows f0.. and up rows I + f0.. of W13[e], R groups of
// 16 rows each reusing one activation fragment per K step.
template <bool kF32, int R>
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
  const int f0 = (fb * 4 + wave) * 16 * R;
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
  const char* wg[R];
  const char* wu[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    wg[r] = w13 + (int64_t)(f0 + 16 * r + m) * H * esz + lane_off;
    wu[r] = w13 + (int64_t)(I + f0 + 16 * r + m) * H * esz + lane_off;
  }
  const char* xr = reinterpret_cast<const char*>(a.a) + src * H * esz + lane_off;
  f32x4 accg[R], accu[R];
#pragma unroll
  for (int r = 0; r < R; ++r) accg[r] = accu[r] = f32x4{0, 0, 0, 0};
  const int kmain = H - H % (kStep * U);
  for (int k0 = 0; k0 < kmain; k0 += kStep * U) {
    Frag32 fg[U][R], fu[U][R], fx[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t o = (int64_t)(k0 + u * kStep) * esz;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        fg[u][r] = load_w(wg[r] + o);
        fu[u][r] = load_w(wu[r] + o);
      }
      fx[u] = load_x(xr + o, xv);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        accg[r] = mma<kF32>(fg[u][r], fx[u], accg[r]);
        accu[r] = mma<kF32>(fu[u][r], fx[u], accu[r]);
      }
  }
  for (int k0 = kmain; k0 < H; k0 += kStep) {
    const int64_t o = (int64_t)k0 * esz;
    const Frag32 fx = load_x(xr + o, xv);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      accg[r] = mma<kF32>(load_w(wg[r] + o), fx, accg[r]);
      accu[r] = mma<kF32>(load_w(wu[r] + o), fx, accu[r]);
    }
  }
  if (xv) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      f32x4 hv;
#pragma unroll
      for (int i = 0; i < 4; ++i) hv[i] = silu_mul(accg[r][i], accu[r][i]);
      store4<kF32>(a.h, (int64_t)(tl.row0 + m) * a.I_max + f0 + 16 * r + kq * 4, hv);
    }
  }
}

// Down projection. Workgroup = (tile, block of 64 R output features of H); wavefront w
// computes R groups of 16 output features, reusing one h fragment per K step.
template <bool kF32, bool kYF32, int R>
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
  const int f0 = (fb * 4 + wave) * 16 * R;
  if (f0 >= H) return;
  const int m = l & 15, kq = l >> 4;
  const int esz = kF32 ? 4 : 2;
  constexpr int kStep = kF32 ? 32 : 64;
  constexpr int kLane = kStep / 4;
  constexpr int U = MOE_STREAM_UNROLL_DN;
  const int64_t lane_off = (int64_t)kq * kLane * esz;
  const bool xv = m < tl.nrows;
  const char* w2 = reinterpret_cast<const char*>(a.bank[bank].w2) + ge * (int64_t)H * I * esz;
  const char* wr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) wr[r] = w2 + (int64_t)(f0 + 16 * r + m) * I * esz + lane_off;
  const char* hr = reinterpret_cast<const char*>(a.h) +
                   (int64_t)(tl.row0 + (xv ? m : 0)) * a.I_max * esz + lane_off;
  f32x4 acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = f32x4{0, 0, 0, 0};
  const int kmain = I - I % (kStep * U);
  for (int k0 = 0; k0 < kmain; k0 += kStep * U) {
    Frag32 fw[U][R], fh[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t o = (int64_t)(k0 + u * kStep) * esz;
#pragma unroll
      for (int r = 0; r < R; ++r) fw[u][r] = load_w(wr[r] + o);
      fh[u] = load_x(hr + o, xv);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = mma<kF32>(fw[u][r], fh[u], acc[r]);
  }
  for (int k0 = kmain; k0 < I; k0 += kStep) {
    const int64_t o = (int64_t)k0 * esz;
    const Frag32 fh = load_x(hr + o, xv);
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = mma<kF32>(load_w(wr[r] + o), fh, acc[r]);
  }
  if (xv) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      store4<kYF32>(a.y, (int64_t)(tl.row0 + m) * H + f0 + 16 * r + kq * 4, acc[r]);
  }
}

}  // namespace

hipError_t launch_ffn_stream(const FfnArgs& a, hipStream_t s, hipEvent_t mid_event) {
  constexpr int RG = MOE_STREAM_ROWS_GU, RD = MOE_STREAM_ROWS_DN;
  const int fb_gu = (a.I_max + kFeatPerWG * RG - 1) / (kFeatPerWG * RG);
  const int fb_dn = (a.H + kFeatPerWG * RD - 1) / (kFeatPerWG * RD);
  const bool f32 = a.wdt == MOE_F32;
  const bool yf32 = a.y_dt == MOE_F32;
  const dim3 blk(256);
  if (f32)
    hipLaunchKernelGGL((k_gateup_stream<true, 1>), dim3(a.max_tiles * ((a.I_max + kFeatPerWG - 1) / kFeatPerWG)), blk, 0, s, a, (a.I_max + kFeatPerWG - 1) / kFeatPerWG);
  else
    hipLaunchKernelGGL((k_gateup_stream<false, RG>), dim3(a.max_tiles * fb_gu), blk, 0, s, a, fb_gu);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (mid_event && (err = hipEventRecord(mid_event, s)) != hipSuccess) return err;
  const int fb_dn1 = (a.H + kFeatPerWG - 1) / kFeatPerWG;
  if (f32 && yf32)
    hipLaunchKernelGGL((k_down_stream<true, true, 1>), dim3(a.max_tiles * fb_dn1), blk, 0, s, a, fb_dn1);
  else if (f32)
    hipLaunchKernelGGL((k_down_stream<true, false, 1>), dim3(a.max_tiles * fb_dn1), blk, 0, s, a, fb_dn1);
  else if (yf32)
    hipLaunchKernelGGL((k_down_stream<false, true, RD>), dim3(a.max_tiles * fb_dn), blk, 0, s, a, fb_dn);
  else
    hipLaunchKernelGGL((k_down_stream<false, false, RD>), dim3(a.max_tiles * fb_dn), blk, 0, s, a, fb_dn);
  return hipGetLastError();
}

}  // namespace moe
