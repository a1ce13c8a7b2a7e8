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
//   (v_mfma_f64_16x16x4_f64). One wavefront per K split and per tile of 16 tokens x 16
//   experts, or of 4 x 2 such tiles for large batches; each lane loads 16 contiguous bytes
//   of each of its token and expert rows, and each loaded fragment feeds 8 MFMAs per tile
//   it belongs to.
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

// K splits are added until about this many wavefronts run (four a SIMD).
constexpr int kRouterWaves = 4096;
// Tokens from which a wavefront takes 4 x 2 tiles (each token fragment feeds 2 tiles,
// each expert fragment 4); below it, one tile.
constexpr int kRouterBigT = 512;

// part[s][t][e] = sum over k in split s of x[t,k] * wr[e,k], in fp64; a wavefront computes
// kRT x kRE tiles of 16 tokens x 16 experts.
template <bool kBF16, int kRT, int kRE>
__global__ void __launch_bounds__(64) k_router_gemm(const void* __restrict__ x,
                                                     const void* __restrict__ wr, int T, int H,
                                                     int E, int klen, double* __restrict__ part) {
  const int l = threadIdx.x;
  const int m = l & 15, kq = l >> 4;
  const int t0 = blockIdx.y * 16 * kRT, e0 = blockIdx.x * 16 * kRE;
  int64_t xrow[kRT], wrow[kRE];
#pragma unroll
  for (int i = 0; i < kRT; ++i) {
    const int t = t0 + 16 * i + m;
    xrow[i] = (int64_t)(t < T ? t : T - 1) * H;
  }
#pragma unroll
  for (int j = 0; j < kRE; ++j) {
    const int e = e0 + 16 * j + m;
    wrow[j] = (int64_t)(e < E ? e : E - 1) * H;
  }
  const int kb = blockIdx.z * klen;
  const int ke = min(H, kb + klen);
  f64x4 acc[kRT][kRE];
#pragma unroll
  for (int i = 0; i < kRT; ++i)
#pragma unroll
    for (int j = 0; j < kRE; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
  for (int k0 = kb; k0 < ke; k0 += 32) {
    const int kk = k0 + kq * 8;
    double a[kRT][8], b[kRE][8];
    if (kk < ke) {
#pragma unroll
      for (int i = 0; i < kRT; ++i) load8<kBF16>(x, xrow[i] + kk, a[i]);
#pragma unroll
      for (int j = 0; j < kRE; ++j) load8<kBF16>(wr, wrow[j] + kk, b[j]);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
#pragma unroll
        for (int i = 0; i < kRT; ++i) a[i][q] = 0.0;
#pragma unroll
        for (int j = 0; j < kRE; ++j) b[j][q] = 0.0;
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int i = 0; i < kRT; ++i)
#pragma unroll
        for (int j = 0; j < kRE; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i][q], b[j][q], acc[i][j], 0, 0, 0);
  }
  // the f64 16x16x4 MFMA leaves D[row kq + 4*r][column m] in lane l, register r
  // (unlike the 16x16 f32-accumulating forms, whose rows are 4*kq + r)
#pragma unroll
  for (int i = 0; i < kRT; ++i)
#pragma unroll
    for (int j = 0; j < kRE; ++j) {
      const int eo = e0 + 16 * j + m;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int to = t0 + 16 * i + kq + 4 * r;
        if (to < T && eo < E) part[((int64_t)blockIdx.z * T + to) * E + eo] = acc[i][j][r];
      }
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

void router_tiles(int32_t T, int* tt, int* te) {
  *tt = T >= kRouterBigT ? 4 : 1;
  *te = T >= kRouterBigT ? 2 : 1;
}

int route_splits(int32_t T, int32_t H, int32_t E, int* klen) {
  int tt, te;
  router_tiles(T, &tt, &te);
  const int64_t tiles = (int64_t)((E + 16 * te - 1) / (16 * te)) * ((T + 16 * tt - 1) / (16 * tt));
  int64_t s = (kRouterWaves + tiles - 1) / (tiles > 0 ? tiles : 1);
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
  int tt, te;
  router_tiles(T, &tt, &te);
  const dim3 g1((E + 16 * te - 1) / (16 * te), (T + 16 * tt - 1) / (16 * tt), S);
  if (x_dt == MOE_BF16 && tt == 4)
    hipLaunchKernelGGL((k_router_gemm<true, 4, 2>), g1, dim3(64), 0, s, x, wr, T, H, E, klen, part);
  else if (x_dt == MOE_BF16)
    hipLaunchKernelGGL((k_router_gemm<true, 1, 1>), g1, dim3(64), 0, s, x, wr, T, H, E, klen, part);
  else if (tt == 4)
    hipLaunchKernelGGL((k_router_gemm<false, 4, 2>), g1, dim3(64), 0, s, x, wr, T, H, E, klen, part);
  else
    hipLaunchKernelGGL((k_router_gemm<false, 1, 1>), g1, dim3(64), 0, s, x, wr, T, H, E, klen, part);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_topk, dim3((T + 3) / 4), dim3(256), 0, s, part, S, T, E, k, (int)fn, scale,
                     bias, topk_idx, topk_w, logits);
  return hipGetLastError();
}

}  // namespace moe
