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
  const char* wg = w13 + (int64_t)(f0 + m) * H * esz;
  const char* wu = w13 + (int64_t)(I + f0 + m) * H * esz;
  const int row = tl.row0 + (m < tl.nrows ? m : tl.nrows - 1);
  const int64_t src = a.a_rowmap ? a.a_rowmap[row] : row;
  const char* xr = reinterpret_cast<const char*>(a.a) + src * H * esz;
  constexpr int kStep = kF32 ? 32 : 64;          // K elements per step
  constexpr int kLane = kStep / 4;               // contiguous elements per lane per step
  f32x4 accg = {0, 0, 0, 0}, accu = {0, 0, 0, 0};
  const int64_t lane_off = (int64_t)kq * kLane * esz;
#pragma unroll 4
  for (int k0 = 0; k0 < H; k0 += kStep) {
    const int64_t o = (int64_t)k0 * esz + lane_off;
    Frag32 fg = load_nt(wg + o);
    Frag32 fu = load_nt(wu + o);
    Frag32 fx = load_c(xr + o);
    if (kF32) {
      accg = mma_f32(fg, fx, accg);
      accu = mma_f32(fu, fx, accu);
    } else {
      accg = mma_bf16(fg, fx, accg);
      accu = mma_bf16(fu, fx, accu);
    }
  }
  if (m < tl.nrows) {
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
  const char* w2 = reinterpret_cast<const char*>(a.bank[bank].w2) + ge * (int64_t)H * I * esz;
  const char* wr = w2 + (int64_t)(f0 + m) * I * esz;
  const int row = tl.row0 + (m < tl.nrows ? m : tl.nrows - 1);
  const char* hr = reinterpret_cast<const char*>(a.h) + (int64_t)row * a.I_max * esz;
  constexpr int kStep = kF32 ? 32 : 64;
  constexpr int kLane = kStep / 4;
  f32x4 acc = {0, 0, 0, 0};
  const int64_t lane_off = (int64_t)kq * kLane * esz;
#pragma unroll 4
  for (int k0 = 0; k0 < I; k0 += kStep) {
    const int64_t o = (int64_t)k0 * esz + lane_off;
    Frag32 fw = load_nt(wr + o);
    Frag32 fh = load_c(hr + o);
    acc = kF32 ? mma_f32(fw, fh, acc) : mma_bf16(fw, fh, acc);
  }
  if (m < tl.nrows) store4<kYF32>(a.y, (int64_t)(tl.row0 + m) * H + f0 + kq * 4, acc);
}

}  // namespace

int32_t ffn_tile_m(moe_dtype wdt, int32_t rows, int32_t groups) {
  (void)wdt;
  (void)rows;
  (void)groups;
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
