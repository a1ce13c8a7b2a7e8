// W4A4 grouped FFN: MXFP4 weights and MXFP4 activations on gfx950's scaled FP4 matrix
// instruction (v_mfma_scale_f32_16x16x128_f8f6f4 with both operands E2M1), the FP4 grouped
// GEMM of "GC-MoE: Overlapping Expert-Parallel Token Dispatch with FP8/FP4 Grouped GEMM via
// CUDA Green Contexts" (key_changes, fourth item) with its operands' E8M0 block scales fed
// to the instruction itself.
//
// Operand layout of one 16 x 16 x 128 instruction: lane (m, q) = (lane % 16, lane / 16)
// holds row m's 32 elements 32 q .. 32 q + 31 as 16 bytes (element 2i in the low nibble of
// byte i) and, in its scale register, the E8M0 scale of that 32-element block; the result
// lane holds D[4 q + i][m]. Activation rows are the A operand, weight rows the B operand.
//
// A workgroup computes 128 rows x 256 weight rows (gate/up: gate and up rows of 128
// features, alternating by 16; 128 x 128 where H or I do not allow 256) with wavefronts of
// 64 x 64; each 128-element K block of both operands (64 B of codes and 4 scale bytes a
// row) goes global -> LDS by DMA through a 3-stage ring (78 KB, two workgroups a CU), the
// kernel's only LDS object. Codes sit in 64-B rows with the 16-B chunk c
// of row r at c ^ ((r >> 2) & 3), so the 16 rows one fragment read touches hit 16 distinct
// bank groups.
//
// The activations are quantised once per token before the gate/up launch
// (k_quant_rows_mxfp4), and the gate/up epilogue quantises h the same way: per 1 x 32
// block, scale 2^e with e = floor(log2(amax)) - 2 (e = 0 for a zero block, clamped to
// [-127, 127]), codes E2M1(v * 2^-e) rounded to nearest even and saturated at 6.
#include "ffn_common.h"

namespace moe {
namespace {

#ifndef MOE_A4_STAGES
#define MOE_A4_STAGES 3
#endif
#ifndef MOE_A4_WGN  // 4: 128 x 256 tiles where the shapes allow; 2: always 128 x 128
#define MOE_A4_WGN 4
#endif

// One thread per 32-element block of a bf16 row: codes [n, H/2] bytes, scales [n, H/32].
__global__ void __launch_bounds__(256) k_quant_rows_mxfp4(const uint16_t* __restrict__ x, int n,
                                                          int H, uint8_t* __restrict__ q,
                                                          uint8_t* __restrict__ qs) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int nb = H / 32;
  if (b >= (int64_t)n * nb) return;
  const int64_t row = b / nb;
  const int blk = (int)(b - row * nb);
  const uint4* src = reinterpret_cast<const uint4*>(x + row * H + blk * 32);
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 w = src[i];
    v[8 * i + 0] = bf16_lo(w.x); v[8 * i + 1] = bf16_hi(w.x);
    v[8 * i + 2] = bf16_lo(w.y); v[8 * i + 3] = bf16_hi(w.y);
    v[8 * i + 4] = bf16_lo(w.z); v[8 * i + 5] = bf16_hi(w.z);
    v[8 * i + 6] = bf16_lo(w.w); v[8 * i + 7] = bf16_hi(w.w);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e = mx_exponent(amax);
  const float inv = exp2i(-e);
  uint32_t wd[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 32; ++i) wd[i >> 3] |= e2m1_code(v[i] * inv) << (4 * (i & 7));
  *reinterpret_cast<uint4*>(q + row * (H / 2) + blk * 16) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  qs[row * nb + blk] = (uint8_t)(e + 127);
}

// LDS offset of logical 16-B chunk c of 64-B code row r.
__device__ __forceinline__ int a4_off(int r, int c) { return r * 64 + ((c ^ ((r >> 2) & 3)) << 4); }

// WGN: wavefronts along the weight rows (2: 128 x 128 tiles, 4 wavefronts; 4: 128 x 256,
// 8 wavefronts).
template <int WGN, bool kGateUp, bool kYF32>
__global__ void __launch_bounds__(128 * WGN, 2) k_w4a4(FfnArgs a, int nb_per_tile) {
  constexpr int S = MOE_A4_STAGES;
  constexpr int TM = 4, TN = 4, WGM = 2, NW = WGM * WGN;
  constexpr int BM = 128, BN = 64 * WGN;
  constexpr int ACODES = BM * 64, BCODES = BN * 64;  // code bytes of each operand a stage
  constexpr int STG = ACODES + BCODES + NW * 256;    // then one 256-B scale slot a wavefront
  constexpr int CPW = (BM + BN) / 16 / NW;           // 1-KB code blocks a wavefront moves
  constexpr int OPS = CPW + 1;                       // DMA instructions per thread a stage
  static_assert((BM + BN) / 16 % NW == 0 && (BM + BN) / 64 <= NW, "DMA shares");
  static_assert(S >= 2 && (S - 2) * OPS < 64, "ring depth");
  __shared__ __attribute__((aligned(1024))) char ring[S * STG];
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  int nb;
  Tile tl;
  if (!xcd_chunked_item(a, nb_per_tile, &nb, &tl)) return;
  const int bank = tl.group < a.E ? 0 : 1;
  const int64_t ge = tl.group < a.E ? tl.group : 0;
  const int I = a.bank[bank].I;
  const int H = a.H;
  const int K = kGateUp ? H : I;
  const int f0 = nb * (kGateUp ? BN / 2 : BN);
  if (f0 >= (kGateUp ? I : H)) return;
  const int64_t wrows = kGateUp ? 2 * I : H;
  const uint8_t* wc = reinterpret_cast<const uint8_t*>(kGateUp ? a.bank[bank].w13 : a.bank[bank].w2) +
                      ge * wrows * (K / 2);
  const uint8_t* ws = reinterpret_cast<const uint8_t*>(kGateUp ? a.bank[bank].w13_scale
                                                               : a.bank[bank].w2_scale) +
                      ge * wrows * (K / 32);
  auto weight_row = [&](int r) {
    if (kGateUp) {
      const int blk = r / (16 * TN), jj = r % (16 * TN), nt = jj >> 4, within = jj & 15;
      const int feat = f0 + blk * (8 * TN) + (nt >> 1) * 16 + within;
      return (nt & 1) ? I + feat : feat;
    }
    return f0 + r;
  };
  auto act_row = [&](int r) -> int64_t {  // source row of tile row r (clamped to the tile)
    const int grow = tl.row0 + (r < tl.nrows ? r : tl.nrows - 1);
    return kGateUp && a.a_rowmap ? a.a_rowmap[grow] : grow;
  };
  // codes: instruction i of wavefront w fills 1-KB block q = NW i + w of the stage's code
  // area (activation rows 16 q .. for q < BM / 16, then weight rows); lane l writes row
  // 16 q + l / 4 of its operand, physical chunk l % 4
  const uint8_t* cp[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int q = NW * i + wave;
    const bool act = q < BM / 16;
    const int r = 16 * (act ? q : q - BM / 16) + (l >> 2);
    const int c = (l & 3) ^ ((r >> 2) & 3);
    if (act) {
      cp[i] = (kGateUp ? a.a_q : reinterpret_cast<const uint8_t*>(a.h)) +
              act_row(r) * (int64_t)(kGateUp ? H / 2 : a.I_max / 2) + c * 16;
    } else {
      cp[i] = wc + (int64_t)weight_row(r) * (K / 2) + c * 16;
    }
  }
  // scales, one dword (4 blocks of 32) a row: wavefront w fetches rows 64 w + l of the
  // activation rows followed by the weight rows (wavefronts past them repeat the last row
  // into their own slot, so that every wavefront issues the same DMA)
  const uint8_t* sp;
  {
    const int r = 64 * wave + l < BM + BN ? 64 * wave + l : BM + BN - 1;
    if (r < BM) {
      sp = (kGateUp ? a.a_xs : a.h_xs) + act_row(r) * (int64_t)(kGateUp ? H / 32 : a.I_max / 32);
    } else {
      sp = ws + (int64_t)weight_row(r - BM) * (K / 32);
    }
  }
  auto issue = [&](int kt) {
    char* st = ring + (kt % S) * STG;
#pragma unroll
    for (int i = 0; i < CPW; ++i) dma16(cp[i] + (int64_t)kt * 64, st + (NW * i + wave) * 1024);
    dma4(sp + (int64_t)kt * 4, st + ACODES + BCODES + wave * 256);
  };
  const int wm = wave % WGM, wn = wave / WGM;
  const bool live = wm * 16 * TM < tl.nrows;
  const int m16 = l & 15, g = l >> 4;
  int arow[TM], brow[TN];
#pragma unroll
  for (int t = 0; t < TM; ++t) arow[t] = wm * (16 * TM) + t * 16 + m16;
#pragma unroll
  for (int t = 0; t < TN; ++t) brow[t] = wn * (16 * TN) + t * 16 + m16;
  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
  const int KT = K / 128;
#pragma unroll
  for (int p = 0; p < S - 1; ++p)
    if (p < KT) issue(p);
  // the K loop, instantiated for wavefronts with rows to multiply and for those without
  // (which still move their share of the DMA and meet every barrier): no branch on the
  // rows inside the loop
  auto kloop = [&](auto live_c) {
    constexpr bool kLive = decltype(live_c)::value != 0;
    for (int kt = 0; kt < KT; ++kt) {
      if (kt + S - 2 < KT) wait_vmcnt<(S - 2) * OPS>();
      else wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      if (kt + S - 1 < KT) issue(kt + S - 1);
      if (!kLive) continue;
      const char* st = ring + (kt % S) * STG;
      i32x8 fa[TM], fb[TN];
      int sa[TM], sb[TN];
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(st + a4_off(arow[t], g));
        fa[t] = i32x8{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
        sa[t] = (int)(*reinterpret_cast<const uint32_t*>(st + ACODES + BCODES + 4 * arow[t]) >> (8 * g));
      }
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(st + ACODES + a4_off(brow[t], g));
        fb[t] = i32x8{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
        sb[t] = (int)(*reinterpret_cast<const uint32_t*>(st + ACODES + BCODES + 4 * (BM + brow[t])) >> (8 * g));
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[i], fb[j], acc[i][j], 4, 4,
                                                                        0, sa[i], 0, sb[j]);
    }
  };
  if (live) kloop(IntC<1>{});
  else kloop(IntC<0>{});
  // lane holds D[row 4 g + i of row tile mt][column m16 of weight tile nt]
#pragma unroll
  for (int mt = 0; mt < TM; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rl = wm * (16 * TM) + mt * 16 + 4 * g + i;
      const bool valid = rl < tl.nrows;  // uniform over the 16 lanes that share a row
      const int64_t row = tl.row0 + rl;
      if (kGateUp) {
        // h of features f0 + 32 wn + 16 p + m16 (p = 0, 1): one 1 x 32 block per row
        float hv[TN / 2];
        float amax = 0.0f;
#pragma unroll
        for (int p = 0; p < TN / 2; ++p) {
          hv[p] = silu_mul(acc[mt][2 * p][i], acc[mt][2 * p + 1][i]);
          amax = fmaxf(amax, fabsf(hv[p]));
        }
#pragma unroll
        for (int s = 1; s < 16; s <<= 1) amax = fmaxf(amax, __shfl_xor(amax, s, 64));
        const int e = mx_exponent(amax);
        const float inv = exp2i(-e);
        const int fb0 = f0 + wn * 32;
#pragma unroll
        for (int p = 0; p < TN / 2; ++p) {
          const uint32_t c = e2m1_code(hv[p] * inv);
          const uint32_t cn = __shfl_xor(c, 1, 64);
          if (valid && (m16 & 1) == 0)
            reinterpret_cast<uint8_t*>(a.h)[row * (a.I_max / 2) + fb0 / 2 + p * 8 + m16 / 2] =
                (uint8_t)(c | (cn << 4));
        }
        if (valid && m16 == 0) a.h_xs[row * (a.I_max / 32) + fb0 / 32] = (uint8_t)(e + 127);
      } else if (valid) {
#pragma unroll
        for (int nt = 0; nt < TN; ++nt) {
          const int64_t o2 = row * H + f0 + wn * (16 * TN) + nt * 16 + m16;
          if (kYF32) reinterpret_cast<float*>(a.y)[o2] = acc[mt][nt][i];
          else reinterpret_cast<uint16_t*>(a.y)[o2] = f32_to_bf16(acc[mt][nt][i]);
        }
      }
    }
  }
}

template <int WGN>
hipError_t launch_w4a4_pair(const FfnArgs& a, hipStream_t s, hipEvent_t mid_event) {
  const int nb_gu = a.I_max / (32 * WGN), nb_dn = a.H / (64 * WGN);
  const dim3 gu(xcd_grid(a.max_tiles, nb_gu)), dn(xcd_grid(a.max_tiles, nb_dn)), blk(128 * WGN);
  hipLaunchKernelGGL((k_w4a4<WGN, true, false>), gu, blk, 0, s, a, nb_gu);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (mid_event && (err = hipEventRecord(mid_event, s)) != hipSuccess) return err;
  if (a.y_dt == MOE_F32)
    hipLaunchKernelGGL((k_w4a4<WGN, false, true>), dn, blk, 0, s, a, nb_dn);
  else
    hipLaunchKernelGGL((k_w4a4<WGN, false, false>), dn, blk, 0, s, a, nb_dn);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_w4a4(const FfnArgs& a, hipStream_t s, hipEvent_t mid_event) {
  // 256 weight rows a workgroup (128 features for gate/up) where every bank allows it
  const bool wide = MOE_A4_WGN == 4 && a.H % 256 == 0 && a.bank[0].I % 128 == 0 &&
                    (!a.has_shared || a.bank[1].I % 128 == 0);
  return wide ? launch_w4a4_pair<4>(a, s, mid_event) : launch_w4a4_pair<2>(a, s, mid_event);
}

hipError_t launch_quant_rows_mxfp4(const void* x, int32_t n, int32_t H, uint8_t* q, uint8_t* qs,
                                   hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t blocks = (int64_t)n * (H / 32);
  hipLaunchKernelGGL(k_quant_rows_mxfp4, dim3((unsigned)((blocks + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const uint16_t*>(x), n, H, q, qs);
  return hipGetLastError();
}

}  // namespace moe
