// Weighted combine: out[t] = sum_j w[t,j] * y[inv_perm[t*k+j]] + shared[t] -- moe_ffn's
// weighted accumulation of the chosen experts' outputs plus the always-active shared
// expert ("Decoding Trillion-Parameter MoE LLMs", section "Routing: Top-K Experts Plus a
// Shared Expert"). A gather, not an atomic scatter: each thread owns 8 consecutive
// elements of one token, sums the k rows in slot order in fp32, adds the shared row and
// rounds once, so the result is deterministic. Loads and stores are 16 B (bf16) or
// 2 x 16 B (fp32) per lane, up to four rows' loads in flight per lane.
#include "moe_internal.h"

namespace moe {
namespace {

#ifndef MOE_COMBINE_GROUP  // slots whose row loads are issued together
#define MOE_COMBINE_GROUP 4
#endif

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

// bf16 expert rows are read with the non-temporal hint (each is read once: e384_fp8's
// combine 0.122 -> 0.096 ms); fp32 rows with cached loads (the hint measured 2% slower on
// r1_prefill's 2.1 GB of fp32 rows).
template <bool kNT, typename V>
__device__ __forceinline__ V ld16(const V* p) {
  if (kNT) return __builtin_nontemporal_load(p);
  return *p;
}

template <bool kYF32>
__device__ __forceinline__ void load8f(const void* base, int64_t off, float* v) {
  if (kYF32) {
    const f32x4v* p = reinterpret_cast<const f32x4v*>(reinterpret_cast<const float*>(base) + off);
    const f32x4v a = ld16<false>(p), b = ld16<false>(p + 1);
    v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3]; v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  } else {
    const u32x4v qv = ld16<true>(reinterpret_cast<const u32x4v*>(reinterpret_cast<const uint16_t*>(base) + off));
    const uint4 q = make_uint4(qv[0], qv[1], qv[2], qv[3]);
    v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
    v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z); v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
  }
}

template <bool kOF32>
__device__ __forceinline__ void store8f(void* base, int64_t off, const float* v) {
  if (kOF32) {
    float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + off);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    uint4 q;
    q.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    q.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
    q.z = (uint32_t)f32_to_bf16(v[4]) | ((uint32_t)f32_to_bf16(v[5]) << 16);
    q.w = (uint32_t)f32_to_bf16(v[6]) | ((uint32_t)f32_to_bf16(v[7]) << 16);
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(base) + off) = q;
  }
}

template <bool kYF32, bool kOF32>
__global__ void __launch_bounds__(256) k_combine(const void* __restrict__ y,
                                                 const int32_t* __restrict__ inv_perm,
                                                 const float* __restrict__ w, int T, int k, int H,
                                                 const void* __restrict__ shared,
                                                 void* __restrict__ out) {
  const int t = blockIdx.x;
  const int h = (blockIdx.y * 256 + threadIdx.x) * 8;
  if (h >= H) return;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  // slots in groups of G: the group's row loads are all issued before the first is used;
  // the sum still runs in slot order
  constexpr int G = MOE_COMBINE_GROUP;
  for (int j0 = 0; j0 < k; j0 += G) {
    const int64_t a = (int64_t)t * k + j0;
    const int nj = k - j0 < G ? k - j0 : G;
    int r[G];
    float wj[G], v[G][8];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      r[j] = j < nj ? inv_perm[a + j] : 0;
      wj[j] = j < nj ? w[a + j] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < G; ++j)
      if (j < nj) load8f<kYF32>(y, (int64_t)r[j] * H + h, v[j]);
#pragma unroll
    for (int j = 0; j < G; ++j)
      if (j < nj) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += wj[j] * v[j][i];
      }
  }
  if (shared) {
    float v[8];
    load8f<kYF32>(shared, (int64_t)t * H + h, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += v[i];
  }
  store8f<kOF32>(out, (int64_t)t * H + h, acc);
}

}  // namespace

hipError_t launch_combine(const void* y, moe_dtype y_dt, const int32_t* inv_perm,
                          const float* topk_w, int32_t T, int32_t k, int32_t H, const void* shared,
                          void* out, moe_dtype out_dt, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid(T, (H / 8 + 255) / 256);
  const bool yf = y_dt == MOE_F32, of = out_dt == MOE_F32;
  if (yf && of)
    hipLaunchKernelGGL((k_combine<true, true>), grid, dim3(256), 0, s, y, inv_perm, topk_w, T, k, H, shared, out);
  else if (yf)
    hipLaunchKernelGGL((k_combine<true, false>), grid, dim3(256), 0, s, y, inv_perm, topk_w, T, k, H, shared, out);
  else if (of)
    hipLaunchKernelGGL((k_combine<false, true>), grid, dim3(256), 0, s, y, inv_perm, topk_w, T, k, H, shared, out);
  else
    hipLaunchKernelGGL((k_combine<false, false>), grid, dim3(256), 0, s, y, inv_perm, topk_w, T, k, H, shared, out);
  return hipGetLastError();
}

}  // namespace moe
