// fp8 grouped-FFN kernel (E4M3 weights with fp32 128 x 128 block scales, activations E4M3 with fp32
// 1 x 128 scales), the FP8 grouped GEMM with fused SwiGLU and re-quantisation of GC-MoE
// (key_changes, fourth item) re-planned for gfx950:
//  - v_mfma_scale_f32_16x16x128_f8f6f4 with unit E8M0 scales computes one 128-wide K block
//    of a 16 x 16 tile exactly; the fp32 block scales (not powers of two, so not foldable
//    into the MFMA's own scale operands) are applied per K block on the VALU:
//    acc += partial * (s_w * s_x[token]).
//  - a workgroup of 8 wavefronts computes 128 rows x 128 output features (one scale block);
//    wavefront w owns features 16 w .. 16 w + 15 with the weights as the MFMA A operand
//    and the tile's <= 128 rows as B. Each K block of both operands and of their scales
//    goes global -> LDS by DMA through a ring (k_fp8 describes it): 3 stages of 49 KB for
//    gate/up (one workgroup a CU, two blocks of weights in flight while one is
//    multiplied), 2 stages of 33 KB for down (two workgroups a CU).
//  - gate/up epilogue: h = SiLU(g) * u in fp32, per-token amax over the workgroup's 128
//    features (wavefront shuffles, then LDS across wavefronts), scale = amax / 448,
//    E4M3 codes of h / scale -- exactly one 1 x 128 quantisation block per workgroup.
#include "ffn_common.h"

namespace moe {
namespace {

#ifndef MOE_F8_STAGES_GU
#define MOE_F8_STAGES_GU 3
#endif
#ifndef MOE_F8_STAGES_DN
#define MOE_F8_STAGES_DN 2
#endif

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

// Quantise rows of a bf16 [n, H] matrix: one workgroup per (row, 16 blocks of 1 x 128), 16
// lanes per block (a workgroup per 2048 elements, so that every row's loads are in flight
// at once).
__global__ void __launch_bounds__(256) k_quant_rows_fp8(const uint16_t* __restrict__ x, int H,
                                                        uint8_t* __restrict__ q,
                                                        float* __restrict__ qs) {
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x;
  const int nblk = H / 128;
  {
    const int b0 = blockIdx.y * 16;
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
  // The K loop for NT 16-row sub-tiles of tokens: NT is fixed per workgroup, so each
  // count gets its own branch-free loop, in which the sub-tiles' LDS reads and MFMAs can
  // be interleaved (a per-sub-tile branch would serialise them).
  auto kloop = [&](auto nt_c) {
    constexpr int NT = decltype(nt_c)::value;
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
      for (int t = 0; t < NT; ++t) {
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
  };
  switch (ntb) {
    case 1: kloop(IntC<1>{}); break;
    case 2: kloop(IntC<2>{}); break;
    case 3: kloop(IntC<3>{}); break;
    case 4: kloop(IntC<4>{}); break;
    case 5: kloop(IntC<5>{}); break;
    case 6: kloop(IntC<6>{}); break;
    case 7: kloop(IntC<7>{}); break;
    default: kloop(IntC<8>{}); break;
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

hipError_t launch_ffn_fp8(const FfnArgs& a, hipStream_t s, hipEvent_t mid_event) {
  const int nb_gu = a.I_max / kF8Feat, nb_dn = a.H / kF8Feat;
  hipLaunchKernelGGL(k_fp8<true>, dim3(a.max_tiles * nb_gu), dim3(512), 0, s, a, nb_gu);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (mid_event && (err = hipEventRecord(mid_event, s)) != hipSuccess) return err;
  hipLaunchKernelGGL(k_fp8<false>, dim3(a.max_tiles * nb_dn), dim3(512), 0, s, a, nb_dn);
  return hipGetLastError();
}

hipError_t launch_quant_rows_fp8(const void* x, int32_t n, int32_t H, uint8_t* q, float* qs,
                                 hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_quant_rows_fp8, dim3(n, (H / 128 + 15) / 16), dim3(256), 0, s,
                     reinterpret_cast<const uint16_t*>(x), H, q, qs);
  return hipGetLastError();
}

}  // namespace moe
