// Grouped SwiGLU FFN for bf16 and fp32 banks whose H or I is a multiple of 8 but not of 64:
// the same per-expert FFN as the other kernel families (moe_ffn's e(x), "Decoding
// Trillion-Parameter MoE LLMs", section "Routing: Top-K Experts Plus a Shared Expert"),
// for the shapes whose K dimension the MFMA kernels' 64-element steps do not tile.
//
// Plain dot products on the vector units, 8 elements (one 16-B bf16 or two 16-B fp32
// loads) a step, summed in fp32 in K order: a workgroup takes one 16-row tile and 16
// output features, thread (r, f) one (row, feature) pair. h stays fp32 between the two
// launches (no bf16 rounding of h, so no residual is needed), y is stored as y_dt asks.
// The workload shapes (H = 7168, I = 2048) never come here; this path exists so that every
// shape the interface admits has a kernel, not for speed.
#include "ffn_common.h"

namespace moe {
namespace {

constexpr int kGenRows = 16;  // rows of a tile (the streaming kernels' tile list)
constexpr int kGenFeat = 16;  // output features a workgroup

// Eight consecutive elements at p (16-B aligned) as fp32.
template <bool kF32>
__device__ __forceinline__ void load8(const void* p, float (&v)[8]) {
  if constexpr (kF32) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
  }
}

// h[row, f] = SiLU(x_row . Wg[f]) * (x_row . Wu[f]) in fp32, for f < I of the tile's bank.
template <bool kF32>
__global__ void __launch_bounds__(kGenRows * kGenFeat) k_gateup_generic(FfnArgs a, int fb_per_tile) {
  const int tile_id = blockIdx.x / fb_per_tile;
  const int fb = blockIdx.x - tile_id * fb_per_tile;
  if (tile_id >= *a.ntiles) return;
  const Tile tl = a.tiles[tile_id];
  const int r = threadIdx.x / kGenFeat, f = fb * kGenFeat + threadIdx.x % kGenFeat;
  const int bank = tl.group < a.E ? 0 : 1;
  const int64_t ge = tl.group < a.E ? tl.group : 0;
  const int I = a.bank[bank].I;
  const int H = a.H;
  if (r >= tl.nrows || f >= I) return;
  const int64_t row = tl.row0 + r;
  const int64_t src = a.a_rowmap ? a.a_rowmap[row] : row;
  constexpr int esz = kF32 ? 4 : 2;
  const char* x = reinterpret_cast<const char*>(a.a) + src * H * esz;
  const char* w13 = reinterpret_cast<const char*>(a.bank[bank].w13) + ge * 2 * I * (int64_t)H * esz;
  const char* wg = w13 + (int64_t)f * H * esz;
  const char* wu = w13 + (int64_t)(I + f) * H * esz;
  float g = 0.0f, u = 0.0f;
  for (int k = 0; k < H; k += 8) {
    float xv[8], gv[8], uv[8];
    load8<kF32>(x + (int64_t)k * esz, xv);
    load8<kF32>(wg + (int64_t)k * esz, gv);
    load8<kF32>(wu + (int64_t)k * esz, uv);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      g = fmaf(xv[j], gv[j], g);
      u = fmaf(xv[j], uv[j], u);
    }
  }
  reinterpret_cast<float*>(a.h)[row * a.I_max + f] = silu_mul(g, u);
}

// y[row, n] = h_row . W2[n] over the bank's I, for n < H; stored as fp32 or bf16.
template <bool kF32, bool kYF32>
__global__ void __launch_bounds__(kGenRows * kGenFeat) k_down_generic(FfnArgs a, int fb_per_tile) {
  const int tile_id = blockIdx.x / fb_per_tile;
  const int fb = blockIdx.x - tile_id * fb_per_tile;
  if (tile_id >= *a.ntiles) return;
  const Tile tl = a.tiles[tile_id];
  const int r = threadIdx.x / kGenFeat, n = fb * kGenFeat + threadIdx.x % kGenFeat;
  const int bank = tl.group < a.E ? 0 : 1;
  const int64_t ge = tl.group < a.E ? tl.group : 0;
  const int I = a.bank[bank].I;
  const int H = a.H;
  if (r >= tl.nrows || n >= H) return;
  const int64_t row = tl.row0 + r;
  constexpr int esz = kF32 ? 4 : 2;
  const float* h = reinterpret_cast<const float*>(a.h) + row * a.I_max;
  const char* w2 = reinterpret_cast<const char*>(a.bank[bank].w2) + (ge * H + n) * (int64_t)I * esz;
  float acc = 0.0f;
  for (int k = 0; k < I; k += 8) {
    float hv[8], wv[8];
    load8<true>(h + k, hv);
    load8<kF32>(w2 + (int64_t)k * esz, wv);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = fmaf(hv[j], wv[j], acc);
  }
  if (kYF32) reinterpret_cast<float*>(a.y)[row * H + n] = acc;
  else reinterpret_cast<uint16_t*>(a.y)[row * H + n] = f32_to_bf16(acc);
}

template <bool kF32>
hipError_t launch_generic(const FfnArgs& a, hipStream_t s, hipEvent_t mid_event) {
  const int fb_gu = (a.I_max + kGenFeat - 1) / kGenFeat, fb_dn = (a.H + kGenFeat - 1) / kGenFeat;
  const dim3 blk(kGenRows * kGenFeat);
  hipLaunchKernelGGL(k_gateup_generic<kF32>, dim3(a.max_tiles * fb_gu), blk, 0, s, a, fb_gu);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (mid_event && (e = hipEventRecord(mid_event, s)) != hipSuccess) return e;
  if (a.y_dt == MOE_F32)
    hipLaunchKernelGGL((k_down_generic<kF32, true>), dim3(a.max_tiles * fb_dn), blk, 0, s, a, fb_dn);
  else
    hipLaunchKernelGGL((k_down_generic<kF32, false>), dim3(a.max_tiles * fb_dn), blk, 0, s, a, fb_dn);
  return hipGetLastError();
}

}  // namespace

bool ffn_generic(moe_dtype wdt, int32_t H, int32_t I_routed, int32_t I_shared) {
  return (wdt == MOE_BF16 || wdt == MOE_F32) &&
         (H % 64 != 0 || I_routed % 64 != 0 || I_shared % 64 != 0);
}

hipError_t launch_ffn_generic(const FfnArgs& a, hipStream_t s, hipEvent_t mid_event) {
  if (a.tile_m != kGenRows) return hipErrorInvalidValue;  // the tile list's height
  return a.wdt == MOE_F32 ? launch_generic<true>(a, s, mid_event)
                          : launch_generic<false>(a, s, mid_event);
}

}  // namespace moe
