// Router: logits, scores, bias-steered top-k selection and renormalised weights.
//
// The router of moe_ffn ("Decoding Trillion-Parameter MoE LLMs: Sparse Architecture and
// Agentic Intelligence", section "Routing: Top-K Experts Plus a Shared Expert") scores
// every token against every expert and keeps the k best, with their weights normalised;
// the per-expert selection bias is the auxiliary-loss-free bias routing named in
// "Chapter 7: Serving Mega-MoE at Scale". Readings taken here: logits are fp64 sums
// rounded once to fp32; scores are computed in fp64; the selection key is fp32(score)
// plus the bias in fp32; equal keys go to the lower expert id; the weights use the
// unbiased scores.
//
// Kernel 1 (k_router_gemm): logits partial sums on the fp64 matrix cores
//   (v_mfma_f64_16x16x4_f64). One wavefront per 16-token x 16-expert tile and K-split;
//   each lane loads 16 contiguous bytes of its token row and of its expert row and feeds
//   8 MFMAs, so loads are 16 B/lane and every input element is read once per tile.
// Kernel 2 (k_topk): one wavefront per token; sums the K-split partials in a fixed order
//   (deterministic), rounds to fp32, scores, and selects k experts by k rounds of a
//   64-lane max over packed (key, expert) 64-bit values.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTopkMaxPerLane = 16;  // E <= 1024

template <bool kBF16>
__device__ __forceinline__ void load8(const void* base, int64_t off, double* v) {
  if (kBF16) {
    uint4 q = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + off);
    v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
    v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z); v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
  } else {
    const float* p = reinterpret_cast<const float*>(base) + off;
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// part[s][t][e] = sum over k in split s of x[t,k] * wr[e,k], in fp64.
template <bool kBF16>
__global__ void __launch_bounds__(64) k_router_gemm(const void* __restrict__ x,
                                                     const void* __restrict__ wr, int T, int H,
                                                     int E, int klen, double* __restrict__ part) {
  const int l = threadIdx.x;
  const int m = l & 15, kq = l >> 4;
  const int t = blockIdx.y * 16 + m;
  const int e = blockIdx.x * 16 + m;
  const int64_t xrow = (int64_t)(t < T ? t : T - 1) * H;
  const int64_t wrow = (int64_t)(e < E ? e : E - 1) * H;
  const int kb = blockIdx.z * klen;
  const int ke = min(H, kb + klen);
  f64x4 acc = {0.0, 0.0, 0.0, 0.0};
  for (int k0 = kb; k0 < ke; k0 += 32) {
    const int kk = k0 + kq * 8;
    double a[8], b[8];
    if (kk < ke) {
      load8<kBF16>(x, xrow + kk, a);
      load8<kBF16>(wr, wrow + kk, b);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) { a[j] = 0.0; b[j] = 0.0; }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a[j], b[j], acc, 0, 0, 0);
  }
  // the f64 16x16x4 MFMA leaves D[row kq + 4*i][column m] in lane l, register i
  // (unlike the 16x16 f32-accumulating forms, whose rows are 4*kq + i)
  const int eo = blockIdx.x * 16 + m;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int to = blockIdx.y * 16 + kq + 4 * i;
    if (to < T && eo < E) part[((int64_t)blockIdx.z * T + to) * E + eo] = acc[i];
  }
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t w = __shfl_xor(v, o, 64);
    v = w > v ? w : v;
  }
  return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Total order on fp32 keys as unsigned integers: larger key -> larger value; -0 == +0;
// NaN -> 0, below every number.
__device__ __forceinline__ uint32_t key_order(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ void __launch_bounds__(256) k_topk(const double* __restrict__ part, int S, int T, int E,
                                              int k, int fn, float scale,
                                              const float* __restrict__ bias,
                                              int32_t* __restrict__ topk_idx,
                                              float* __restrict__ topk_w,
                                              float* __restrict__ logits) {
  const int l = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float lg[kTopkMaxPerLane];
  double sc[kTopkMaxPerLane];
  uint64_t key[kTopkMaxPerLane];
#pragma unroll
  for (int i = 0; i < kTopkMaxPerLane; ++i) {
    const int e = i * 64 + l;
    lg[i] = 0.0f;
    if (e < E) {
      double s = 0.0;
      // unrolled so that the loads of a group of partials are in flight together; the
      // sum still runs in split order
#pragma unroll 8
      for (int p = 0; p < S; ++p) s += part[((int64_t)p * T + t) * E + e];
      lg[i] = (float)s;
      if (logits) logits[(int64_t)t * E + e] = lg[i];
    }
  }
  if (fn == MOE_SIGMOID) {
#pragma unroll
    for (int i = 0; i < kTopkMaxPerLane; ++i) sc[i] = 1.0 / (1.0 + exp(-(double)lg[i]));
  } else {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < kTopkMaxPerLane; ++i)
      if (i * 64 + l < E) mx = fmaxf(mx, lg[i]);
    mx = wave_max_f32(mx);
    double sum = 0.0;
#pragma unroll
    for (int i = 0; i < kTopkMaxPerLane; ++i) {
      sc[i] = (i * 64 + l < E) ? exp((double)lg[i] - (double)mx) : 0.0;
      sum += sc[i];
    }
    sum = wave_sum_f64(sum);
#pragma unroll
    for (int i = 0; i < kTopkMaxPerLane; ++i) sc[i] = sc[i] / sum;
  }
#pragma unroll
  for (int i = 0; i < kTopkMaxPerLane; ++i) {
    const int e = i * 64 + l;
    if (e < E) {
      float kf = (float)sc[i];
      if (bias) kf = kf + bias[e];
      key[i] = ((uint64_t)key_order(kf) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
    } else {
      key[i] = 0ull;
    }
  }
  int sel[16];
  for (int r = 0; r < k; ++r) {
    uint64_t best = 0ull;
#pragma unroll
    for (int i = 0; i < kTopkMaxPerLane; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
    sel[r] = e;
#pragma unroll
    for (int i = 0; i < kTopkMaxPerLane; ++i)
      if (i * 64 + l == e) key[i] = 0ull;
  }
  // ascending expert order (k <= 16: insertion sort, identical in every lane)
  for (int a = 1; a < k; ++a) {
    int v = sel[a], b = a - 1;
    while (b >= 0 && sel[b] > v) { sel[b + 1] = sel[b]; --b; }
    sel[b + 1] = v;
  }
  double chosen[16];
  double tot = 0.0;
  for (int r = 0; r < k; ++r) {
    const int e = sel[r];
    double v = 0.0;
#pragma unroll
    for (int i = 0; i < kTopkMaxPerLane; ++i)
      if (i == (e >> 6)) v = sc[i];
    v = __shfl(v, e & 63, 64);
    chosen[r] = v;
    tot += v;
  }
  if (l < k) {
    double v = 0.0;
    int e = 0;
    for (int r = 0; r < k; ++r)
      if (r == l) { v = chosen[r]; e = sel[r]; }
    topk_idx[(int64_t)t * k + l] = e;
    topk_w[(int64_t)t * k + l] = (float)((double)scale * v / tot);
  }
}

int route_splits(int32_t T, int32_t H, int32_t E, int* klen) {
  const int64_t tiles = (int64_t)((E + 15) / 16) * ((T + 15) / 16);
  int64_t s = (1024 + tiles - 1) / (tiles > 0 ? tiles : 1);
  int64_t smax = H / 256 > 1 ? H / 256 : 1;
  if (s > smax) s = smax;
  if (s < 1) s = 1;
  int len = (int)((H + s - 1) / s);
  len = (len + 31) / 32 * 32;
  *klen = len;
  return (H + len - 1) / len;
}

}  // namespace

size_t route_ws_bytes(int32_t T, int32_t H, int32_t E) {
  int klen;
  int S = route_splits(T, H, E, &klen);
  size_t part = (size_t)S * T * E * sizeof(double);
  return (part + 255) / 256 * 256;
}

hipError_t launch_route(const void* x, moe_dtype x_dt, const void* wr, const float* bias,
                        int32_t T, int32_t H, int32_t E, int32_t k, moe_score_fn fn, float scale,
                        int32_t* topk_idx, float* topk_w, float* logits, void* ws, hipStream_t s) {
  if (T == 0) return hipSuccess;
  int klen;
  int S = route_splits(T, H, E, &klen);
  double* part = reinterpret_cast<double*>(ws);
  dim3 g1((E + 15) / 16, (T + 15) / 16, S);
  if (x_dt == MOE_BF16)
    hipLaunchKernelGGL(k_router_gemm<true>, g1, dim3(64), 0, s, x, wr, T, H, E, klen, part);
  else
    hipLaunchKernelGGL(k_router_gemm<false>, g1, dim3(64), 0, s, x, wr, T, H, E, klen, part);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_topk, dim3((T + 3) / 4), dim3(256), 0, s, part, S, T, E, k, (int)fn, scale,
                     bias, topk_idx, topk_w, logits);
  return hipGetLastError();
}

}  // namespace moe
