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
// For bf16 inputs from 512 tokens on, when the logits are not asked for, kernels 1f and
// 2f (below) first select from bf16 matrix-core sums with a proven error bound, and
// kernels 1 and 2 then route only the tokens whose selection that bound leaves open.
#include "ffn_common.h"  // LDS layout and DMA helpers of the tiled kernels

namespace moe {
namespace {

constexpr int kTopkMaxPerLane = 16;  // E <= 1024
// The top-k kernels are instantiated for 1, 2, 4, 8 and 16 experts a lane; a launch takes
// the smallest that covers E (registers and guards scale with it).
#define MOE_TOPK_LAUNCH(KERNEL, E_, ...)                                         \
  do {                                                                          \
    const int npl_ = ((E_) + 63) / 64;                                          \
    if (npl_ <= 1) hipLaunchKernelGGL((KERNEL<1>), __VA_ARGS__);                \
    else if (npl_ <= 2) hipLaunchKernelGGL((KERNEL<2>), __VA_ARGS__);           \
    else if (npl_ <= 4) hipLaunchKernelGGL((KERNEL<4>), __VA_ARGS__);           \
    else if (npl_ <= 8) hipLaunchKernelGGL((KERNEL<8>), __VA_ARGS__);           \
    else hipLaunchKernelGGL((KERNEL<kTopkMaxPerLane>), __VA_ARGS__);            \
  } while (0)

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

// K splits are added until about this many wavefronts run (two a SIMD; 1024, 4096 and
// 8192 measured slower on the route step at T = 128 and T = 8192).
#ifndef MOE_ROUTER_WAVES
#define MOE_ROUTER_WAVES 2048
#endif
constexpr int kRouterWaves = MOE_ROUTER_WAVES;
// Tokens from which a wavefront takes 4 x 2 tiles (each token fragment feeds 2 tiles,
// each expert fragment 4); below it, one tile.
constexpr int kRouterBigT = 512;

// part[s][t][e] = sum over k in split s of x[t,k] * wr[e,k], in fp64; a wavefront computes
// kRT x kRE tiles of 16 tokens x 16 experts.
// K splits for the n listed tokens: up to kFbMaxSplits (and H / 256), as far as the
// partial-sum buffer (cap rows of E) allows; the partials are [splits][n][E].
constexpr int kFbMaxSplits = 16;
__device__ __forceinline__ int fb_splits(int n, int64_t cap, int H, int* klen) {
  int64_t sp = H / 256 < kFbMaxSplits ? H / 256 : kFbMaxSplits;
  if (n > 0 && sp > cap / n) sp = cap / n;
  if (sp < 1) sp = 1;
  int len = (int)((H + sp - 1) / sp);
  len = (len + 31) / 32 * 32;
  *klen = len;
  return (H + len - 1) / len;
}

// With a token list (list, cnt): row t of the tile is token list[t], for t < *cnt, with
// its own K splits (fb_splits; cap rows of partials).
template <bool kBF16, int kRT, int kRE>
__global__ void __launch_bounds__(64) k_router_gemm(const void* __restrict__ x,
                                                     const void* __restrict__ wr, int T, int H,
                                                     int E, int klen, double* __restrict__ part,
                                                     const int32_t* __restrict__ list,
                                                     const int32_t* __restrict__ cnt, int64_t cap) {
  const int l = threadIdx.x;
  const int m = l & 15, kq = l >> 4;
  const int e0 = blockIdx.x * 16 * kRE;
  const int nrows = list ? *cnt : T;
  int64_t stride = T;
  if (list) {
    if ((int)blockIdx.z >= fb_splits(nrows, cap, H, &klen)) return;
    stride = nrows;
  }
  // a grid over all tiles without a list; with one, a few rows of workgroups step through
  // the listed tokens' tiles
  for (int ty = blockIdx.y;; ty += gridDim.y) {
    const int t0 = ty * 16 * kRT;
    if (t0 >= nrows) return;
    int64_t xrow[kRT], wrow[kRE];
#pragma unroll
    for (int i = 0; i < kRT; ++i) {
      const int t = t0 + 16 * i + m;
      const int r = t < nrows ? t : nrows - 1;
      xrow[i] = (int64_t)(list ? list[r] : r) * H;
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
          if (to < nrows && eo < E) part[((int64_t)blockIdx.z * stride + to) * E + eo] = acc[i][j][r];
        }
      }
    if (!list) return;
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

// With a token list (list, cnt): wavefront p < *cnt handles token list[p], whose partials
// are row p of part.
template <int NPL>  // experts per lane: E <= 64 NPL
__global__ void __launch_bounds__(256) k_topk(const double* __restrict__ part, int S, int T, int E,
                                              int k, int fn, float scale,
                                              const float* __restrict__ bias,
                                              int32_t* __restrict__ topk_idx,
                                              float* __restrict__ topk_w,
                                              float* __restrict__ logits,
                                              const int32_t* __restrict__ list,
                                              const int32_t* __restrict__ cnt, int H, int64_t cap) {
  const int l = threadIdx.x & 63;
  const int p0 = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n = list ? *cnt : T;
  if (p0 >= n) return;
  const int t = list ? list[p0] : p0;
  int64_t stride = T;
  if (list) {
    int kl;
    S = fb_splits(n, cap, H, &kl);
    stride = n;
  }
  float lg[NPL];
  double sc[NPL];
  uint64_t key[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = i * 64 + l;
    lg[i] = 0.0f;
    if (e < E) {
      double s = 0.0;
      // unrolled so that the loads of a group of partials are in flight together; the
      // sum still runs in split order
#pragma unroll 8
      for (int p = 0; p < S; ++p) s += part[((int64_t)p * stride + p0) * E + e];
      lg[i] = (float)s;
      if (logits) logits[(int64_t)t * E + e] = lg[i];
    }
  }
  if (fn == MOE_SIGMOID) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) sc[i] = 1.0 / (1.0 + exp(-(double)lg[i]));
  } else {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (i * 64 + l < E) mx = fmaxf(mx, lg[i]);
    mx = wave_max_f32(mx);
    double sum = 0.0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      sc[i] = (i * 64 + l < E) ? exp((double)lg[i] - (double)mx) : 0.0;
      sum += sc[i];
    }
    sum = wave_sum_f64(sum);
#pragma unroll
    for (int i = 0; i < NPL; ++i) sc[i] = sc[i] / sum;
  }
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
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
    for (int i = 0; i < NPL; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
    sel[r] = e;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
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
    for (int i = 0; i < NPL; ++i)
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

// ------------------------------------------------------------- certified fast router
//
// Used for bf16 inputs when the fp32 logits themselves are not asked for.
// Kernel 0f (k_row_norms2) sums the squares of every router row in fp64.
// Kernel 1f (k_router_lds) multiplies on the bf16 matrix cores: each 64-element K block
// of a (token, expert) dot product is summed in fp32 by two chained
// v_mfma_f32_16x16x32_bf16 (a product of two bf16 values is exact in fp32), and the block
// sums are added in fp64, one partial sum per K split.
// Kernel 2f (k_topk_fast) adds the splits, sums the squares of the token's row in fp64,
// bounds the distance of every sum from the exact dot product, turns the bound into an
// interval for each expert's key (key and score are non-decreasing in the logit:
// sigmoid; for softmax, in the own logit and non-increasing in the others), and takes the
// k experts of the largest approximate keys only if every chosen interval lies strictly
// above every other one. The exact keys then choose the same k experts, and their exact
// fp64 dot products give the fp32 logits and the weights. Where the intervals overlap,
// the same wavefront takes exact logits of the few experts that can still be chosen (at
// most 16) and chooses among them (k_topk_fast describes how). A token that this leaves
// undecided (more candidates, keys equal to within the bounds, non-finite values) is
// appended to a list that the exact kernels 1 and 2 then route.
//
// The bound. A block sum of 64 exact products formed with fp32 additions, in whatever
// order the matrix core adds and as long as each addition errs by at most 2^-23 of its
// result, lies within 64 * 2^-23 of the sum of the products' magnitudes from the exact
// block sum; kCertRel doubles that. Over all blocks, and by Cauchy-Schwarz,
// |sum - exact| <= kCertRel ||x_t|| ||w_e||. Inputs or products in the subnormal range
// may be flushed to zero: such a product is below 2^-126 max(|x_h|, |w_h|, 1), covered
// by H 2^-126 (||x_t|| + ||w_e|| + 1). The fp64 additions (errors near 2^-50 relative)
// are covered by the factor 1 + 2^-30.
constexpr double kCertRel = 0x1p-16;  // 2 * 64 * 2^-23
constexpr int kXcds = 8;              // MI355X: workgroups dealt to 8 XCDs round-robin
// rows of 16-token tiles in the grid of the exact kernel over the token list
constexpr int kListTileRows = 64;

// Kernel 1f: a workgroup of 4 x 2 wavefronts takes 128 tokens x 128 experts (a wavefront
// 32 x 64), and each 64-element K block of the token rows and of the router rows goes
// global -> LDS by DMA through an S-stage ring (the LDS layout and slot map of the tiled
// expert GEMM), so every token row is fetched once per 128 experts and every router row
// once per 128 tokens. Items (K split, token tile, expert tile), expert tile fastest, are
// cut into kXcds contiguous chunks; chunk c runs on the workgroups the dispatcher deals to
// XCD c (blockIdx mod kXcds), so that the expert tiles reading one token tile share an L2.
#ifndef MOE_RT_STAGES
#define MOE_RT_STAGES 2
#endif
#ifndef MOE_RT_WPS  // wavefronts a SIMD the register budget must allow
#define MOE_RT_WPS 2
#endif
constexpr int kRtWgt = 4, kRtWge = 2;                          // wavefronts along tokens, experts
constexpr int kRtTokens = kRtWgt * 32, kRtExperts = kRtWge * 64;  // 128 x 128

__global__ void __launch_bounds__(64 * kRtWgt * kRtWge, MOE_RT_WPS) k_router_lds(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int H, int E,
    int klen, int ntt, int net, int nz, double* __restrict__ part,
    int32_t* __restrict__ cnt) {
  constexpr int TM = 2, TN = 4, NW = kRtWgt * kRtWge, S = MOE_RT_STAGES;
  constexpr int XST = kRtTokens * 128, STG = XST + kRtExperts * 128;  // bytes a stage
  constexpr int CX = kRtTokens / (NW * 8), CW = kRtExperts / (NW * 8);  // DMA ops a thread
  constexpr int OPS = CX + CW;
  static_assert(CX >= 1 && CW >= 1 && S >= 2 && (S - 2) * OPS < 64, "router ring");
  __shared__ __attribute__((aligned(1024))) char smem[S * STG];
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int m16 = l & 15, g = l >> 4;
  const int nitems = nz * ntt * net;
  const int chunk = (nitems + kXcds - 1) / kXcds;
  const int slot = blockIdx.x / kXcds;
  const int item = (blockIdx.x % kXcds) * chunk + slot;
  if (blockIdx.x == 0 && tid == 0) *cnt = 0;
  if (slot >= chunk || item >= nitems) return;
  const int ex = item % net, ty = (item / net) % ntt, z = item / (net * ntt);
  const int t0 = ty * kRtTokens, e0 = ex * kRtExperts;
  const int wm = wave % kRtWgt, wn = wave / kRtWgt;
  // DMA sources: 1-KB block q = NW i + wave of each tile (rows and 16-B chunks of dma_slot)
  const char* xs[CX];
  const char* ws[CW];
#pragma unroll
  for (int i = 0; i < CX; ++i) {
    int r, c;
    dma_slot(NW * i + wave, l, &r, &c);
    const int t = t0 + r;
    xs[i] = reinterpret_cast<const char*>(x) + (int64_t)(t < T ? t : T - 1) * H * 2 + c * 16;
  }
#pragma unroll
  for (int i = 0; i < CW; ++i) {
    int r, c;
    dma_slot(NW * i + wave, l, &r, &c);
    const int e = e0 + r;
    ws[i] = reinterpret_cast<const char*>(wr) + (int64_t)(e < E ? e : E - 1) * H * 2 + c * 16;
  }
  const int kb0 = z * klen / 64;
  const int KT = (min(H, z * klen + klen) - z * klen) / 64;
  auto issue = [&](int kt) {
    char* st = smem + (kt % S) * STG;
    const int64_t o = (int64_t)(kb0 + kt) * 128;
#pragma unroll
    for (int i = 0; i < CX; ++i) dma16(xs[i] + o, st + (NW * i + wave) * 1024);
#pragma unroll
    for (int i = 0; i < CW; ++i) dma16(ws[i] + o, st + XST + (NW * i + wave) * 1024);
  };
  f64x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int p = 0; p < S - 1; ++p)
    if (p < KT) issue(p);
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + S - 2 < KT) wait_vmcnt<(S - 2) * OPS>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (kt + S - 1 < KT) issue(kt + S - 1);
    const char* st = smem + (kt % S) * STG;
    // one fp32 chain per 16 x 16 tile over the block's two k-steps, then added in fp64
    f32x4 p[TM][TN];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 fa[TM], fb[TN];
      const int c = 2 * g + ks;
#pragma unroll
      for (int t = 0; t < TM; ++t)
        fa[t] = *reinterpret_cast<const uint4*>(st + lds_off(wm * 32 + 16 * t + m16, c));
#pragma unroll
      for (int t = 0; t < TN; ++t)
        fb[t] = *reinterpret_cast<const uint4*>(st + XST + lds_off(wn * 64 + 16 * t + m16, c));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          p[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, fa[i]), __builtin_bit_cast(bf16x8, fb[j]),
              ks ? p[i][j] : f32x4{0, 0, 0, 0}, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] += (double)p[i][j][r];
  }
  // the f32-accumulating 16x16 MFMA leaves D[row 4 g + r][column m] in lane l, register r
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int eo = e0 + wn * 64 + 16 * j + m16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int to = t0 + wm * 32 + 16 * i + 4 * g + r;
        if (to < T && eo < E) part[((int64_t)z * T + to) * E + eo] = acc[i][j][r];
      }
    }
}

// Squared norms of the router rows, in fp64 (one wavefront a row, a fixed summation order).
__global__ void __launch_bounds__(256) k_row_norms2(const uint16_t* __restrict__ w, int n, int H,
                                                    double* __restrict__ out) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
  if (row >= n) return;
  const uint16_t* p = w + (int64_t)row * H;
  double v = 0.0;
#pragma unroll 8  // the loads of eight chunks in flight together; the sum keeps its order
  for (int h = 8 * l; h < H; h += 512) {
    const uint4 q = *reinterpret_cast<const uint4*>(p + h);
    const double v0 = bf16_lo(q.x), v1 = bf16_hi(q.x), v2 = bf16_lo(q.y), v3 = bf16_hi(q.y);
    const double v4 = bf16_lo(q.z), v5 = bf16_hi(q.z), v6 = bf16_lo(q.w), v7 = bf16_hi(q.w);
    v += ((v0 * v0 + v1 * v1) + (v2 * v2 + v3 * v3)) + ((v4 * v4 + v5 * v5) + (v6 * v6 + v7 * v7));
  }
  v = wave_sum_f64(v);
  if (l == 0) out[row] = v;
}

__device__ __forceinline__ double wave_max_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t w = __shfl_xor(v, o, 64);
    v = w < v ? w : v;
  }
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t w = __shfl_xor(v, o, 64);
    v = w > v ? w : v;
  }
  return v;
}

// At most this many candidate experts are refined in k_topk_fast (two passes of eight).
constexpr int kRefineMax = 16;
#ifndef MOE_LOGIT_UNROLL  // chunks of the exact dot products whose loads go out together
#define MOE_LOGIT_UNROLL 1   // (2: the same speed with registers spilled at 3 workgroups a CU)
#endif
#ifndef MOE_TOPK_FAST_WPS  // wavefronts a SIMD that k_topk_fast's register budget must allow
#define MOE_TOPK_FAST_WPS 2  // (3: route step 7-10 us longer at e384_fp8 and r1_prefill)
#endif

// Exact logits of token row xr against router rows ids[0..8): fp64 dot products of the
// bf16 values (each product exact), rounded once to fp32. Lane l takes the 8-element
// chunks l, l + 64, ... of x and of the eight rows, whose loads of one chunk are issued
// together.
__device__ __forceinline__ void exact_logits8(const uint16_t* __restrict__ xr,
                                              const uint16_t* __restrict__ wr, int H,
                                              const int* ids, int l, double* out) {
  int64_t woff[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) woff[r] = (int64_t)ids[r] * H;
  double dot[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) dot[r] = 0.0;
#pragma unroll MOE_LOGIT_UNROLL  // the sums keep their order whatever the unrolling
  for (int h = 8 * l; h < H; h += 512) {
    const uint4 a = *reinterpret_cast<const uint4*>(xr + h);
    uint4 b[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) b[r] = *reinterpret_cast<const uint4*>(wr + woff[r] + h);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      double d = dot[r];
      d += (double)bf16_lo(a.x) * (double)bf16_lo(b[r].x);
      d += (double)bf16_hi(a.x) * (double)bf16_hi(b[r].x);
      d += (double)bf16_lo(a.y) * (double)bf16_lo(b[r].y);
      d += (double)bf16_hi(a.y) * (double)bf16_hi(b[r].y);
      d += (double)bf16_lo(a.z) * (double)bf16_lo(b[r].z);
      d += (double)bf16_hi(a.z) * (double)bf16_hi(b[r].z);
      d += (double)bf16_lo(a.w) * (double)bf16_lo(b[r].w);
      d += (double)bf16_hi(a.w) * (double)bf16_hi(b[r].w);
      dot[r] = d;
    }
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) out[r] = (double)(float)wave_sum_f64(dot[r]);
}

template <int NPL>  // experts per lane: E <= 64 NPL
__global__ void __launch_bounds__(256, MOE_TOPK_FAST_WPS) k_topk_fast(
    const double* __restrict__ part, const double* __restrict__ nw2s, int S, int T, int H, int E,
    int k, int fn, float scale,
    const float* __restrict__ bias, const uint16_t* __restrict__ x,
    const uint16_t* __restrict__ wr, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int32_t* __restrict__ list, int32_t* __restrict__ cnt) {
  // per-wavefront slots for the refinement of a token whose choice the bounds leave open
  __shared__ int r_id[4][kRefineMax];
  __shared__ double r_lg[4][kRefineMax], r_t[4][kRefineMax];
  __shared__ uint64_t r_lo[4][kRefineMax], r_hi[4][kRefineMax];
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + w;
  if (t >= T) return;
  // ||x_t||^2 in fp64 from the token's row (its chunks are read again, from cache, for the
  // exact dot products below)
  const uint16_t* xr = x + (int64_t)t * H;
  double nx2 = 0.0;
#pragma unroll 7  // the row's loads in flight together (H = 7168: all 14); the sum keeps its order
  for (int h = 8 * l; h < H; h += 512) {
    const uint4 q = *reinterpret_cast<const uint4*>(xr + h);
    const double v0 = bf16_lo(q.x), v1 = bf16_hi(q.x), v2 = bf16_lo(q.y), v3 = bf16_hi(q.y);
    const double v4 = bf16_lo(q.z), v5 = bf16_hi(q.z), v6 = bf16_lo(q.w), v7 = bf16_hi(q.w);
    nx2 += ((v0 * v0 + v1 * v1) + (v2 * v2 + v3 * v3)) + ((v4 * v4 + v5 * v5) + (v6 * v6 + v7 * v7));
  }
  const double nx = sqrt(wave_sum_f64(nx2));
  const double tiny = (double)H * 0x1p-126;
  float lo[NPL], hi[NPL], mid[NPL];
  bool fin = true;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = i * 64 + l;
    lo[i] = hi[i] = mid[i] = 0.0f;
    if (e < E) {
      double sum = 0.0;
#pragma unroll 8
      for (int p = 0; p < S; ++p) sum += part[((int64_t)p * T + t) * E + e];
      const double nw = sqrt(nw2s[e]);
      const double beta = (kCertRel * nx * nw + tiny * (nx + nw + 1.0)) * (1.0 + 0x1p-30);
      fin = fin && __builtin_isfinite(sum) && __builtin_isfinite(beta);
      // the exact logit fp32(exact sum) lies in [lo, hi] (rounding is monotone)
      lo[i] = (float)(sum - beta);
      hi[i] = (float)(sum + beta);
      mid[i] = (float)sum;
    }
  }
  bool certified = __all(fin);
  uint32_t klo[NPL], khi[NPL];
  uint64_t key[NPL];
  if (certified) {
    // The interval keys use fp32 exp, whose results (with the add and the division) are
    // within 2^-20 of the exact values; kWiden moves each bound outward by more than
    // that. exp of an fp32 difference d also carries the rounding of d, |d| 2^-24
    // relative, which lo_exp / hi_exp add per term. The middle keys only order the
    // candidates.
    constexpr double kWiden = 0x1p-17;
    auto lo_exp = [&](float d) { return (double)expf(d) * (1.0 - kWiden - fabs((double)d) * 0x1p-22); };
    auto hi_exp = [&](float d) { return (double)expf(d) * (1.0 + kWiden + fabs((double)d) * 0x1p-22); };
    // softmax over intervals: p_e is smallest with its own logit low and the others high,
    // largest the other way round (sums of the exponentials first, then each key)
    float mh = 0.0f, mm = 0.0f;
    double Alo = 0.0, Ahi = 0.0, Am = 0.0;
    const double rel = (double)E * 0x1p-50;  // rounding of the fp64 sums, relative
    if (fn != MOE_SIGMOID) {
      float fh = -INFINITY, fm = -INFINITY;
#pragma unroll
      for (int i = 0; i < NPL; ++i)
        if (i * 64 + l < E) { fh = fmaxf(fh, hi[i]); fm = fmaxf(fm, mid[i]); }
      mh = wave_max_f32(fh);
      mm = wave_max_f32(fm);
#pragma unroll
      for (int i = 0; i < NPL; ++i)
        if (i * 64 + l < E) {
          Alo += fmax(lo_exp(lo[i] - mh), 0.0);
          Ahi += hi_exp(hi[i] - mh);
          Am += (double)expf(mid[i] - mm);
        }
      Alo = wave_sum_f64(Alo);
      Ahi = wave_sum_f64(Ahi);
      Am = wave_sum_f64(Am);
    }
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = i * 64 + l;
      klo[i] = khi[i] = 0u;
      key[i] = 0ull;
      if (e >= E) continue;
      double slo, shi, smid;
      if (fn == MOE_SIGMOID) {
        slo = (double)(1.0f / (1.0f + expf(-lo[i]))) * (1.0 - kWiden);
        shi = (double)(1.0f / (1.0f + expf(-hi[i]))) * (1.0 + kWiden);
        smid = 1.0f / (1.0f + expf(-mid[i]));
      } else {
        // lo[i] <= hi[i] <= mh, so the exponentials are at most 1 (up to rounding)
        const double alo = fmax(lo_exp(lo[i] - mh), 0.0), ahi = hi_exp(hi[i] - mh);
        const double rest_hi = (Ahi - ahi) + Ahi * rel;
        const double rest_lo = fmax((Alo - alo) - Alo * rel, 0.0);
        slo = alo / (alo + rest_hi) * (1.0 - kWiden);
        shi = ahi > 0.0 ? ahi / (ahi + rest_lo) * (1.0 + kWiden) : 0.0;
        smid = (double)expf(mid[i] - mm) / Am;
      }
      float a = (float)slo, b = (float)shi, c = (float)smid;
      if (bias) { a = a + bias[e]; b = b + bias[e]; c = c + bias[e]; }
      klo[i] = key_order(a);
      khi[i] = key_order(b);
      key[i] = ((uint64_t)key_order(c) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
    }
  }
  int sel[16];
  double lg[16];  // exact logits of the chosen experts, in the order of sel
  if (certified) {
    uint32_t chosen = 0u;  // bit i: expert 64 i + l is chosen
    for (int r = 0; r < k; ++r) {
      uint64_t best = 0ull;
#pragma unroll
      for (int i = 0; i < NPL; ++i) best = key[i] > best ? key[i] : best;
      best = wave_max_u64(best);
      const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
      sel[r] = e;
#pragma unroll
      for (int i = 0; i < NPL; ++i)
        if (i * 64 + l == e) { key[i] = 0ull; chosen |= 1u << i; }
    }
    uint32_t min_in = 0xFFFFFFFFu, max_out = 0u;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      if (i * 64 + l >= E) continue;
      if (chosen >> i & 1u) min_in = klo[i] < min_in ? klo[i] : min_in;
      else max_out = khi[i] > max_out ? khi[i] : max_out;
    }
    certified = wave_min_u32(min_in) > wave_max_u32(max_out);
  }
  if (certified) {
    for (int a = 1; a < k; ++a) {
      int v = sel[a], b = a - 1;
      while (b >= 0 && sel[b] > v) { sel[b + 1] = sel[b]; --b; }
      sel[b + 1] = v;
    }
    // exact logits of the chosen experts
    for (int r0 = 0; r0 < k; r0 += 8) {
      int ids[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) ids[r] = r0 + r < k ? sel[r0 + r] : sel[r0];
      double v[8];
      exact_logits8(xr, wr, H, ids, l, v);
#pragma unroll
      for (int r = 0; r < 8; ++r)
        if (r0 + r < k) lg[r0 + r] = v[r];
    }
  } else {
    // Not separated. The experts that can be among the k largest exact keys are those
    // whose upper key bound reaches L, the k-th largest lower bound: k experts have exact
    // keys >= L, so an expert whose key lies below L is beaten k times. With at most
    // kRefineMax of them (the candidates), their exact logits are computed and the k are
    // chosen among them on key bounds that hold the exact path's keys: exact for sigmoid;
    // for softmax the normaliser (a sum over all experts, the others' logits known to
    // their intervals) is known to an interval, which is all that widens them. A token
    // whose choice these bounds do not settle goes to the list for the exact kernels.
    bool done = false;
    if (__all(fin)) {
      uint64_t kk[NPL];
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        const int e = i * 64 + l;
        kk[i] = e < E ? ((uint64_t)klo[i] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e) : 0ull;
      }
      uint64_t kth = 0ull;
      for (int r = 0; r < k; ++r) {
        uint64_t best = 0ull;
#pragma unroll
        for (int i = 0; i < NPL; ++i) best = kk[i] > best ? kk[i] : best;
        kth = wave_max_u64(best);
#pragma unroll
        for (int i = 0; i < NPL; ++i)
          if (kk[i] == kth) kk[i] = 0ull;
      }
      const uint32_t L = (uint32_t)(kth >> 32);
      uint64_t cm[NPL];
      int nc = 0;
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        cm[i] = __ballot(i * 64 + l < E && khi[i] >= L);
        nc += __popcll(cm[i]);
      }
      if (nc <= kRefineMax) {
        // the candidates' data (uniform) in this wavefront's slots, candidates in
        // increasing id order; written by lane 0 and read back by every lane
        int* rid = r_id[w];
        double* rlg = r_lg[w];
        uint64_t* rlo = r_lo[w];
        uint64_t* rhi = r_hi[w];
        double* rt = r_t[w];
        {
          uint64_t m[NPL];
#pragma unroll
          for (int i = 0; i < NPL; ++i) m[i] = cm[i];
          for (int j = 0; j < nc; ++j) {
            int id = -1;
#pragma unroll
            for (int i = 0; i < NPL; ++i)
              if (id < 0 && m[i] != 0ull) {
                id = i * 64 + __builtin_ctzll(m[i]);
                m[i] &= m[i] - 1ull;
              }
            if (l == 0) rid[j] = id;
          }
        }
        __builtin_amdgcn_wave_barrier();
        for (int j0 = 0; j0 < nc; j0 += 8) {
          int ids[8];
#pragma unroll
          for (int r = 0; r < 8; ++r) ids[r] = rid[j0 + r < nc ? j0 + r : j0];
          double v[8];
          exact_logits8(xr, wr, H, ids, l, v);
#pragma unroll
          for (int r = 0; r < 8; ++r)
            if (l == 0 && j0 + r < nc) rlg[j0 + r] = v[r];
        }
        __builtin_amdgcn_wave_barrier();
        // key bounds of the candidates as 64-bit (key, ~id) values
        double shi = 1.0;
        if (fn == MOE_SIGMOID) {
          for (int j = 0; j < nc; ++j) {
            float kf = (float)(1.0 / (1.0 + exp(-rlg[j])));
            if (bias) kf = kf + bias[rid[j]];
            const uint64_t v = ((uint64_t)key_order(kf) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)rid[j]);
            if (l == 0) { rlo[j] = v; rhi[j] = v; }
          }
        } else {
          // the exact path's max is the largest exact logit, a candidate's; its sum of
          // exp(logit - max) over all experts lies in [slo, shi]: the candidates' terms as
          // it computes them, the others' from their logit bounds, widened by 2^-40 for
          // the rounding of exp and of the sums in any order
          double mx = -INFINITY;
          for (int j = 0; j < nc; ++j) mx = fmax(mx, rlg[j]);
          double slo = 0.0;
          shi = 0.0;
          int before = 0;  // candidates in the slots before this lane's expert of slot i
#pragma unroll
          for (int i = 0; i < NPL; ++i) {
            const int e = i * 64 + l;
            const uint64_t below = l ? cm[i] & (~0ull >> (64 - l)) : 0ull;
            if (e < E) {
              if (cm[i] >> l & 1ull) {
                const double tc = exp(rlg[before + __popcll(below)] - mx);
                slo += tc;
                shi += tc;
              } else {
                slo += exp((double)lo[i] - mx);
                shi += exp((double)hi[i] - mx);
              }
            }
            before += __popcll(cm[i]);
          }
          slo = wave_sum_f64(slo) * (1.0 - 0x1p-40);
          shi = wave_sum_f64(shi) * (1.0 + 0x1p-40);
          for (int j = 0; j < nc; ++j) {
            const double tc = exp(rlg[j] - mx);
            float a = (float)(tc / shi), b = (float)(tc / slo);
            if (bias) { a = a + bias[rid[j]]; b = b + bias[rid[j]]; }
            const uint64_t id = (uint64_t)(0xFFFFFFFFu - (uint32_t)rid[j]);
            if (l == 0) {
              rt[j] = tc;
              rlo[j] = ((uint64_t)key_order(a) << 32) | id;
              rhi[j] = ((uint64_t)key_order(b) << 32) | id;
            }
          }
        }
        __builtin_amdgcn_wave_barrier();
        // Softmax without bias: every key is fp32(t / S) with the same S, so a candidate
        // whose t exceeds another's by more than a factor 1 + 2^-22 (with keys above the
        // subnormal range) has the strictly larger key whatever S is; the choice is then
        // made by t.
        const bool by_t = fn != MOE_SIGMOID && !bias;
        uint32_t cho = 0u;
        for (int r = 0; r < k; ++r) {
          int bj = -1;
          for (int j = 0; j < nc; ++j) {
            if (cho >> j & 1u) continue;
            // candidates are in increasing id order: a later one wins only if larger
            if (bj < 0 || (by_t ? rt[j] > rt[bj] : rlo[j] > rlo[bj])) bj = j;
          }
          if (bj >= 0) cho |= 1u << bj;
        }
        // settled if the weakest chosen candidate certainly beats the strongest other
        uint64_t min_in = ~0ull, max_out = 0ull;
        double tmin = INFINITY, tmax = 0.0;
        for (int j = 0; j < nc; ++j) {
          if (cho >> j & 1u) {
            min_in = rlo[j] < min_in ? rlo[j] : min_in;
            if (by_t) tmin = fmin(tmin, rt[j]);
          } else {
            max_out = rhi[j] > max_out ? rhi[j] : max_out;
            if (by_t) tmax = fmax(tmax, rt[j]);
          }
        }
        const bool sep = __builtin_popcount(cho) == k &&
                         (min_in > max_out ||
                          (by_t && tmin > tmax * (1.0 + 0x1p-22) && tmax / shi >= 0x1p-100));
        if (sep) {
          int r = 0;
          for (int j = 0; j < nc; ++j)
            if (cho >> j & 1u) {
              sel[r] = rid[j];
              lg[r] = rlg[j];
              ++r;
            }
          done = true;
        }
      }
    }
    if (!done) {
      if (l == 0) list[atomicAdd(cnt, 1)] = t;
      return;
    }
  }
  double mx = -INFINITY;
  for (int r = 0; r < k; ++r) mx = fmax(mx, lg[r]);
  // weights from the unbiased scores of the chosen experts (softmax: renormalised over
  // the chosen, i.e. the softmax of their logits)
  double sc[16];
  double tot = 0.0;
  for (int r = 0; r < k; ++r) {
    sc[r] = fn == MOE_SIGMOID ? 1.0 / (1.0 + exp(-lg[r])) : exp(lg[r] - mx);
    tot += sc[r];
  }
  if (l < k) {
    double v = 0.0;
    int e = 0;
    for (int r = 0; r < k; ++r)
      if (r == l) { v = sc[r]; e = sel[r]; }
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

namespace {
size_t al256(size_t b) { return (b + 255) / 256 * 256; }
}  // namespace

// part [S][T][E] f64, then (certified fast router) the squared norms of the router rows
// [E] in f64, the token list [T] int32 and its count.
size_t route_ws_bytes(int32_t T, int32_t H, int32_t E) {
  int klen;
  int S = route_splits(T, H, E, &klen);
  return al256((size_t)S * T * E * sizeof(double)) + al256((size_t)E * sizeof(double)) +
         al256((size_t)T * sizeof(int32_t)) + 256;
}

hipError_t launch_route(const void* x, moe_dtype x_dt, const void* wr, const float* bias,
                        int32_t T, int32_t H, int32_t E, int32_t k, moe_score_fn fn, float scale,
                        int32_t* topk_idx, float* topk_w, float* logits, void* ws, hipStream_t s) {
  if (T == 0) return hipSuccess;
  int klen;
  int S = route_splits(T, H, E, &klen);
  double* part = reinterpret_cast<double*>(ws);
  if (x_dt == MOE_BF16 && logits == nullptr && H % 64 == 0 && T >= kRouterBigT) {
    char* w = reinterpret_cast<char*>(ws) + al256((size_t)S * T * E * sizeof(double));
    double* nw2 = reinterpret_cast<double*>(w);
    w += al256((size_t)E * sizeof(double));
    int32_t* list = reinterpret_cast<int32_t*>(w);
    int32_t* cnt = reinterpret_cast<int32_t*>(w + al256((size_t)T * sizeof(int32_t)));
    // K splits of the LDS kernel: about kRouterWaves wavefronts, at most S (the buffers)
    const int net = (E + kRtExperts - 1) / kRtExperts, ntt = (T + kRtTokens - 1) / kRtTokens;
    const int64_t tiles = (int64_t)net * ntt * (kRtWgt * kRtWge);
    int64_t sf = (kRouterWaves + tiles - 1) / tiles;
    sf = sf < 1 ? 1 : sf > S ? S : sf;
    int flen = (int)((H + sf - 1) / sf);
    flen = (flen + 63) / 64 * 64;
    const int SF = (H + flen - 1) / flen;
    const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
    const uint16_t* wb = reinterpret_cast<const uint16_t*>(wr);
    hipLaunchKernelGGL(k_row_norms2, dim3((E + 3) / 4), dim3(256), 0, s, wb, E, H, nw2);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int nblk = (SF * ntt * net + kXcds - 1) / kXcds * kXcds;  // whole rounds of kXcds
    hipLaunchKernelGGL(k_router_lds, dim3(nblk), dim3(64 * kRtWgt * kRtWge), 0, s, xb, wb, T, H, E,
                       flen, ntt, net, SF, part, cnt);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    MOE_TOPK_LAUNCH(k_topk_fast, E, dim3((T + 3) / 4), dim3(256), 0, s, part, nw2, SF, T, H, E, k,
                       (int)fn, scale, bias, xb, wb, topk_idx, topk_w, list, cnt);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    // the listed tokens, exactly: the grid covers T tokens, wavefronts past the count exit
    const int64_t cap = (int64_t)S * T;
    const dim3 gx((E + 15) / 16, (T + 15) / 16 < kListTileRows ? (T + 15) / 16 : kListTileRows,
                  kFbMaxSplits);
    hipLaunchKernelGGL((k_router_gemm<true, 1, 1>), gx, dim3(64), 0, s, x, wr, T, H, E, klen, part,
                       list, cnt, cap);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    MOE_TOPK_LAUNCH(k_topk, E, dim3((T + 3) / 4), dim3(256), 0, s, part, S, T, E, k, (int)fn, scale,
                       bias, topk_idx, topk_w, nullptr, list, cnt, H, cap);
    return hipGetLastError();
  }
  int tt, te;
  router_tiles(T, &tt, &te);
  const dim3 g1((E + 16 * te - 1) / (16 * te), (T + 16 * tt - 1) / (16 * tt), S);
  if (x_dt == MOE_BF16 && tt == 4)
    hipLaunchKernelGGL((k_router_gemm<true, 4, 2>), g1, dim3(64), 0, s, x, wr, T, H, E, klen, part,
                       nullptr, nullptr, 0);
  else if (x_dt == MOE_BF16)
    hipLaunchKernelGGL((k_router_gemm<true, 1, 1>), g1, dim3(64), 0, s, x, wr, T, H, E, klen, part,
                       nullptr, nullptr, 0);
  else if (tt == 4)
    hipLaunchKernelGGL((k_router_gemm<false, 4, 2>), g1, dim3(64), 0, s, x, wr, T, H, E, klen, part,
                       nullptr, nullptr, 0);
  else
    hipLaunchKernelGGL((k_router_gemm<false, 1, 1>), g1, dim3(64), 0, s, x, wr, T, H, E, klen, part,
                       nullptr, nullptr, 0);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  MOE_TOPK_LAUNCH(k_topk, E, dim3((T + 3) / 4), dim3(256), 0, s, part, S, T, E, k, (int)fn, scale,
                     bias, topk_idx, topk_w, logits, nullptr, nullptr, H, 0);
  return hipGetLastError();
}

}  // namespace moe
