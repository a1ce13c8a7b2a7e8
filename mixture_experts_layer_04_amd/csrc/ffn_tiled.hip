// LDS-tiled grouped-FFN kernel (many rows per expert, e.g. prefill), for bf16 and MXFP4
// weights: the grouped GEMM with fused SwiGLU of "GC-MoE: Overlapping Expert-Parallel
// Token Dispatch with FP8/FP4 Grouped GEMM via CUDA Green Contexts" (key_changes, fourth
// item), planned for gfx950.
//
// A workgroup computes a tile of rows x weight rows (gate/up: the gate and up rows of
// half as many features, alternating by 16, so that each lane holds gate and up of the
// same (row, feature) and SwiGLU is applied in registers) with a WGM x WGN grid of
// wavefronts, each (16 TM) x (16 TN) with v_mfma_f32_16x16x32_bf16: for bf16, 256 x 256
// with 16 wavefronts of 64 x 64 (one workgroup a CU, four wavefronts a SIMD) where H and
// I allow, else 128 x 128 with 4 wavefronts (two workgroups a CU); for MXFP4 128 x 256
// with 4 wavefronts of 64 x 128. Per flop the 256 x 256 tile moves half the bytes from
// L2 into LDS, which bounds these kernels. The K blocks (64 elements) go
// from global memory straight into LDS with global_load_lds (no register staging),
// through an S-stage ring, so that each block has S-1 blocks of MFMA work to hide
// behind. A lane's fragment of a K block is the 32 contiguous bytes at 32 (lane / 16)
// in both operands (K index 16 (lane / 16) + 8 ks + j for k-step ks).
//
// LDS layout of a K block (128 B per row): each 16-row group takes 2 KB = eight 256-B
// lines; line j holds row j in its low 128 B and row 8 + j in its high 128 B, and the
// 16-B chunk c of row r sits at chunk c ^ (r & 7). Measured on MI355X, this lets the
// fragment reads of 16 consecutive rows at one chunk run at the full LDS rate
// (~250 B/clk/CU) where padded or plainly swizzled rows reach half of it. A wavefront's
// DMA writes 1 KB contiguously (16 B per lane, lane order), i.e. 4 + 4 rows of a group,
// and each lane's global address absorbs the layout.
//
// bf16 weights: the gate/up epilogue writes h as bf16 plus its MXFP4-coded residual
// (ffn_common.h), and the down launch stages the residual with its activation rows (32 B
// of E2M1 codes and a scale dword a row, laid out as the MXFP4 weight rows are), decodes
// each residual fragment as it is read and multiplies it with the same weight fragment:
// two MFMAs per fragment pair. MXFP4 weights keep a plain bf16 h.
#include "ffn_common.h"

namespace moe {
namespace {

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
#ifndef MOE_T2_STAGES_B_GU  // weight-ring stages of the bf16 gate/up launch
#define MOE_T2_STAGES_B_GU 2
#endif
#ifndef MOE_T2_STAGES_B_DN  // weight-ring stages of the bf16 down launch (73 KB with the
#define MOE_T2_STAGES_B_DN 2  // residual of h in the activation stages: 2 WGs a CU)
#endif
#ifndef MOE_T2_MX_STAGES
#define MOE_T2_MX_STAGES 2
#endif
#ifndef MOE_T2_MX_TN
#define MOE_T2_MX_TN 8
#endif
#ifndef MOE_T2_WAVES_PER_SIMD
#define MOE_T2_WAVES_PER_SIMD 2
#endif
// bf16 with 256 x 256 tiles: 4 x 4 wavefronts of 4 x 4 MFMA tiles; a 2-stage activation
// ring and a 2-stage weight ring, 128 KB (gate/up) or 146 KB (down, whose activation
// stages also hold h's residual) of LDS
#ifndef MOE_T2B_STAGES_B_GU
#define MOE_T2B_STAGES_B_GU 2
#endif
#ifndef MOE_T2B_STAGES_B_DN  // down: 2 weight stages beside 2 activation stages that also
#define MOE_T2B_STAGES_B_DN 2  // carry h's residual (146 KB)
#endif
static_assert(4 * 16 * 4 == kTiledMB && 4 * 16 * 4 == kTiledNB, "tile shape of the tile list");
// waves a SIMD that the register budget must allow: a 16-wavefront workgroup puts four on
// each SIMD of its CU, and two 8-wavefront workgroups a CU do the same
constexpr int waves_per_simd(int nw) { return nw >= 8 ? 4 : MOE_T2_WAVES_PER_SIMD; }
constexpr int kT2M = MOE_T2_WGM * 16 * MOE_T2_TM, kT2N = MOE_T2_WGN * 16 * MOE_T2_TN;
static_assert(kT2M == kTiledM && kT2N == kTiledN, "tile shape of the tile list");

// Workgroup of WGM x WGN wavefronts; each wavefront computes (16 TM) x (16 TN).
// kMX: MXFP4 weights. A K block of a weight row is then 32 B of E2M1 codes plus 2 E8M0
// scale bytes; the ring stages the codes (32 B a row: the 8-B quarter u of row r at
// quarter u ^ 2 ((r >> 3) & 1), which spreads the 64-bit fragment reads of 16 rows over
// all banks) and 4 scale bytes a row (those of K blocks kt & ~1 and (kt & ~1) + 1, one
// aligned dword), and fragments are decoded to bf16 in registers as they are read.
template <int TM, int TN, int WGM, int WGN, int S, int SB, bool kGateUp, bool kYF32, bool kMX>
__global__ void __launch_bounds__(64 * WGM * WGN, waves_per_simd(WGM * WGN)) k_tiled2(FfnArgs a, int nb_per_tile) {
  constexpr int NW = WGM * WGN;
  constexpr int BM = WGM * 16 * TM, BN = WGN * 16 * TN;
  constexpr int BSTAGE = kMX ? BN * 32 + BN * 4 : BN * 128;  // weight bytes of a stage
  // bf16 weights: h carries an MXFP4 residual; the down launch stages it with the A rows
  constexpr bool kLo = !kMX;
  constexpr bool kALo = kLo && !kGateUp;
  constexpr int AHI = BM * 128;                // activation (h) bytes of a stage
  constexpr int ALO = kALo ? BM * 32 : 0;      // residual codes of a stage
  constexpr int ASTAGE = AHI + ALO + (kALo ? BM * 4 : 0);  // + their scale dwords
  // residual: each wavefront moves UPWA 16-B units of codes (one instruction, LPWA lanes)
  // and the scale dwords of SPWA rows
  constexpr int UPWA = BM * 2 / NW;
  constexpr int LPWA = UPWA;
  constexpr int SPWA = BM / NW;
  constexpr int CAL = kALo ? 2 : 0;            // DMA instructions per thread: codes + scales
  static_assert(!kALo || (BM * 2 % NW == 0 && UPWA <= 64 && UPWA % 2 == 0 && SPWA <= 64),
                "residual DMA rounds");
  static_assert(!kLo || TN == 4, "a lane's gate/up features span one 32-feature block");
  constexpr int RPI = NW * 8;                  // LDS rows filled per DMA instruction round
  constexpr int CA = BM / RPI;                 // DMA instructions per thread per K block: A,
  // MXFP4: each wavefront moves its UPW 16-B units of a stage's codes (CB instructions,
  // the last one with LPW lanes) and its SPW rows' scale dwords (one instruction)
  constexpr int UPW = BN * 2 / NW;
  constexpr int CB = kMX ? (UPW + 63) / 64 : BN / RPI;  // B,
  constexpr int LPW = UPW - 64 * (CB - 1);
  constexpr int CS = kMX ? 1 : 0;                       // MXFP4 scales
  constexpr int SPW = BN / NW;
  static_assert(BM % RPI == 0 && BN % RPI == 0 && BM % 16 == 0, "tile rows per DMA round");
  static_assert(!kMX || (BN * 2 % NW == 0 && UPW % 2 == 0 && BN % NW == 0 && SPW <= 64),
                "MXFP4 DMA rounds");
  // activation ring (S stages), then weight ring (SB stages): the weights, which mostly
  // come from HBM, may be requested further ahead than the activations, mostly L2 hits
  __shared__ __attribute__((aligned(1024))) char smem[S * ASTAGE + SB * BSTAGE];
  // the wavefront index as a uniform (scalar) value: the DMA destinations derive from it
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  // Work items (tile, weight block) are cut into 8 equal contiguous chunks, chunk x run by
  // the workgroups that the dispatcher deals to XCD x (blockIdx = x mod 8; xcd_chunked_item),
  // so that each XCD's L2 serves the items that share data. Inside a chunk the items of a block
  // of up to kTileBlock row tiles of one group run weight block by weight block, the
  // block's row tiles side by side: they read the same weight rows at the same time, and
  // the items that read one activation tile are at most kTileBlock apart.
  int nb;
  Tile tl;
  if (!xcd_chunked_item(a, nb_per_tile, &nb, &tl)) return;
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
      // lane l of instruction i: 16-B unit UPW w + 64 i + l of the codes, i.e. row
      // (unit / 2) and physical half l % 2 of its 32-B slice (idle lanes repeat lane 0)
      const int u = UPW * wave + 64 * i + ((i + 1 < CB || l < LPW) ? l : 0);
      const int r = u >> 1;
      const int lh = (u & 1) ^ ((r >> 3) & 1);
      bg[i] = wbase + weight_row(r) * wrow_bytes + lh * 16;
    } else {
      int r, cc;
      dma_slot(NW * i + wave, l, &r, &cc);
      bg[i] = wbase + weight_row(r) * wrow_bytes + cc * 16;
    }
  }
  // residual of h (down, bf16): lane l of wavefront w moves 16-B unit UPWA w + l of the
  // codes (row unit / 2, physical half l % 2 swizzled as for MXFP4 weight rows) and, if
  // l < SPWA, the scale dword of row SPWA w + l
  const uint8_t* alg = nullptr;
  const uint8_t* asg = nullptr;
  if (kALo) {
    const int u = UPWA * wave + (l < LPWA ? l : 0);
    const int r = u >> 1;
    const int lh = (u & 1) ^ ((r >> 3) & 1);
    const int grow = tl.row0 + (r < tl.nrows ? r : tl.nrows - 1);
    alg = a.h_lo + (int64_t)grow * (a.I_max / 2) + lh * 16;
    const int rs = SPWA * wave + (l < SPWA ? l : 0);
    const int grs = tl.row0 + (rs < tl.nrows ? rs : tl.nrows - 1);
    asg = a.h_lo_s + (int64_t)grs * lo_sstride(a.I_max);
  }
  if (kMX) {
    // lanes l < SPW of wavefront w fetch the scale dword of B-tile row SPW w + l
    const uint8_t* sbase = reinterpret_cast<const uint8_t*>(kGateUp ? a.bank[bank].w13_scale
                                                                    : a.bank[bank].w2_scale) +
                           ge * wrows * (K / 32);
    sg = sbase + weight_row(SPW * wave + (l < SPW ? l : 0)) * (int64_t)(K / 32);
  }
  auto issue_a = [&](int kt) {
    char* st = smem + (kt % S) * ASTAGE;
#pragma unroll
    for (int i = 0; i < CA; ++i) dma16(ag[i] + (int64_t)kt * 128, st + (NW * i + wave) * 1024);
    if (kALo) {
      if (l < LPWA) dma16(alg + (int64_t)kt * 32, st + AHI + UPWA * wave * 16);
      if (l < SPWA) dma4(asg + (kt & ~1) * 2, st + AHI + ALO + wave * (SPWA * 4));
    }
  };
  auto issue_b = [&](int kt) {
    char* st = smem + S * ASTAGE + (kt % SB) * BSTAGE;
    if (kMX) {
#pragma unroll
      for (int i = 0; i < CB; ++i)
        if (i + 1 < CB || l < LPW) dma16(bg[i] + (int64_t)kt * 32, st + (UPW * wave + 64 * i) * 16);
      if (l < SPW) dma4(sg + (kt & ~1) * 2, st + BN * 32 + wave * (SPW * 4));
    } else {
#pragma unroll
      for (int i = 0; i < CB; ++i) dma16(bg[i] + (int64_t)kt * 128, st + (NW * i + wave) * 1024);
    }
  };
  const int wm = wave % WGM, wn = wave / WGM;
  const bool live = wm * 16 * TM < tl.nrows;
  const int m16 = l & 15, g = l >> 4;
  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
  const int KT = K / 64;  // 64-element K blocks (128 B of bf16 a row)
  // This lane's fragment rows are arow0 + 16 t (A) and brow0 + 16 t (B). Adding 16 t leaves
  // a row's low four bits alone, so in every LDS layout here row tile t's read is the
  // first one's plus a constant (2048 t in lds_off's, 512 t in 32-B code rows, 64 t in
  // scale dwords): one per-lane base offset per read kind, the rest immediates.
  const int arow0 = wm * (16 * TM) + m16, brow0 = wn * (16 * TN) + m16;
  const int aoff[2] = {lds_off(arow0, 2 * g), lds_off(arow0, 2 * g + 1)};  // per k-step
  const int boff[2] = {lds_off(brow0, 2 * g), lds_off(brow0, 2 * g + 1)};
  // 32-B E2M1 code rows (MXFP4 weights; h's residual): this lane's 8-B quarter g, swizzled
  const int bq = brow0 * 32 + 8 * (g ^ (((brow0 >> 3) & 1) << 1));
  const int lq0 = AHI + arow0 * 32 + 8 * (g ^ (((arow0 >> 3) & 1) << 1));
  // Step i issues A(i + S - 1), then B(i + SB - 1); the steps before the loop issue the
  // blocks >= 0 of steps -(max(S, SB) - 1) .. -1. Block kt has landed once no more DMA
  // instructions are outstanding than were issued after the later of A(kt) and B(kt).
  constexpr int OA = CA + CAL, OB = CB + CS, SL = S > SB ? S : SB;
  constexpr int AFTER = S < SB ? OB + (S - 2) * (OA + OB) : (SB - 2) * (OA + OB);
  static_assert(S >= 2 && SB >= 2 && AFTER < 64, "ring depths");
#pragma unroll
  for (int p = 1 - SL; p < 0; ++p) {
    if (p + S - 1 >= 0 && p + S - 1 < KT) issue_a(p + S - 1);
    if (p + SB - 1 >= 0 && p + SB - 1 < KT) issue_b(p + SB - 1);
  }
  // The K loop, instantiated for wavefronts with rows to multiply (kLive) and for those
  // whose rows all lie past the tile's last row, which only move their share of the DMA
  // and meet every barrier. (Deciding this inside the loop, per K block, measured 2-7%
  // slower; so did further instantiations per count of live 16-row sub-tiles, with the DMA
  // of empty sub-tiles skipped.)
  auto kloop = [&](auto live_c) {
    constexpr bool kLive = decltype(live_c)::value != 0;
    for (int kt = 0; kt < KT; ++kt) {
      if (kt + SL - 2 < KT) wait_vmcnt<AFTER>();
      else wait_vmcnt<0>();
      // A plain barrier, not __syncthreads(): its fence would wait for every outstanding
      // DMA of the ring. The wait above already covers this thread's part of block kt.
      __builtin_amdgcn_s_barrier();
      if (kt + S - 1 < KT) issue_a(kt + S - 1);
      if (kt + SB - 1 < KT) issue_b(kt + SB - 1);
      if (!kLive) continue;
      const char* cur = smem + (kt % S) * ASTAGE;                 // activations of block kt
      const char* curb = smem + S * ASTAGE + (kt % SB) * BSTAGE;  // weights of block kt
      // MXFP4: this lane's 16 codes (elements 16 g .. 16 g + 15 of the K block) and scale
      uint2 wq[kMX ? TN : 1];
      float wsc[kMX ? TN : 1];
      // the scale byte of this lane's 16 elements within a row's scale dword
      const int sbyte = (kt & 1) * 2 + (g >> 1);
      if (kMX) {
        const char* q = curb + bq;
        const char* sc = curb + BN * 32 + 4 * brow0 + sbyte;
#pragma unroll
        for (int t = 0; t < TN; ++t) {
          // two 32-bit reads: with one 64-bit read the compiler makes it wait for all DMA
          wq[t].x = *reinterpret_cast<const uint32_t*>(q + 512 * t);
          wq[t].y = *reinterpret_cast<const uint32_t*>(q + 512 * t + 4);
          wsc[t] = e8m0_f32_fast(*reinterpret_cast<const uint8_t*>(sc + 64 * t));
        }
      }
      // bf16 down: the block scale of this lane's 16 residual elements of each A row (the
      // writer emits codes 0..254 only; code 0, a scale of 2^-127 for residuals below
      // 2^-125, decodes to 0 here)
      float lsc[kALo ? TM : 1];
      if (kALo) {
        const char* sc = cur + AHI + ALO + 4 * arow0 + sbyte;
#pragma unroll
        for (int t = 0; t < TM; ++t)
          lsc[t] = __uint_as_float((uint32_t)*reinterpret_cast<const uint8_t*>(sc + 64 * t) << 23);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 fa[TM], fb[TN];
        uint32_t lq[kALo ? TM : 1];  // the residual's 8 codes of k-step ks, each A row
        const char* pa = cur + aoff[ks];
#pragma unroll
        for (int t = 0; t < TM; ++t) fa[t] = *reinterpret_cast<const bf16x8*>(pa + 2048 * t);
        if (kALo) {
          const char* q = cur + lq0 + 4 * ks;
#pragma unroll
          for (int t = 0; t < TM; ++t) lq[t] = *reinterpret_cast<const uint32_t*>(q + 512 * t);
        }
        const char* pb = curb + boff[ks];
#pragma unroll
        for (int t = 0; t < TN; ++t) {
          if (kMX) fb[t] = e2m1x8_bf16(ks ? wq[t].y : wq[t].x, wsc[t]);
          else fb[t] = *reinterpret_cast<const bf16x8*>(pb + 2048 * t);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        if (kALo) {
          // then the residual: each A row tile's fragment decoded just before its MFMAs
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            const bf16x8 fl = e2m1x8_bf16(lq[i], lsc[i]);
#pragma unroll
            for (int j = 0; j < TN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fl, fb[j], acc[i][j], 0, 0, 0);
          }
        }
      }
    }
  };
  if (live) kloop(IntC<1>{});
  else kloop(IntC<0>{});
#pragma unroll
  for (int mt = 0; mt < TM; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rl = wm * (16 * TM) + mt * 16 + 4 * g + i;
      if (rl >= tl.nrows) continue;
      const int64_t row = tl.row0 + rl;
      if (kGateUp && kLo) {
        // h = hi + lo: hi bf16; lo as MXFP4 over the lane group's 32-feature block (the 16
        // lanes of group g hold row rl's features fb + 16 p + m16, p = 0, 1)
        const int fb = f0 + wn * (8 * TN);
        float lo[TN / 2];
        float am = 0.0f;
#pragma unroll
        for (int p = 0; p < TN / 2; ++p) {
          const float hv = silu_mul(acc[mt][2 * p][i], acc[mt][2 * p + 1][i]);
          reinterpret_cast<uint16_t*>(a.h)[row * a.I_max + fb + p * 16 + m16] = split_bf16(hv, &lo[p]);
          am = fmaxf(am, fabsf(lo[p]));
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
        const int e = mx_exponent(am);
        const float inv = exp2i(-e);
#pragma unroll
        for (int p = 0; p < TN / 2; ++p) {
          const uint32_t cd = e2m1_code(lo[p] * inv);
          const uint32_t nb2 = __shfl_xor(cd, 1, 64);  // the neighbouring feature's code
          if ((m16 & 1) == 0)
            a.h_lo[row * (a.I_max / 2) + (fb + p * 16 + m16) / 2] = (uint8_t)(cd | (nb2 << 4));
        }
        if (m16 == 0) a.h_lo_s[row * lo_sstride(a.I_max) + fb / 32] = (uint8_t)(e + 127);
      } else if (kGateUp) {
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

// MXFP4 may take a wider weight tile (MOE_T2_MX_TN column tiles a wavefront): its K
// slices are a quarter of bf16's, so the ring still leaves room for two workgroups a CU.
constexpr int kMXN = MOE_T2_WGN * 16 * MOE_T2_MX_TN;

// SB: weight-ring stages of the gate/up launch, SBD of the down launch; TND x WGND: the
// down launch's column tiles a wavefront and wavefronts along the weight rows (the same
// 16 TN WGN weight rows a workgroup, the same row tiles)
template <int TM, int TN, int WGM, int WGN, int S, int SB, int SBD, bool kMX, int TND = TN,
          int WGND = WGN>
hipError_t launch_tiled_pair(const FfnArgs& a, hipStream_t s, hipEvent_t mid_event) {
  constexpr int BN = WGN * 16 * TN;
  static_assert(WGND * 16 * TND == BN, "both launches take the same weight block");
  const int nb_gu = a.I_max / (BN / 2), nb_dn = a.H / BN;
  // whole rounds of 8 workgroups, so that every chunk's last item has a workgroup
  const dim3 gu(xcd_grid(a.max_tiles, nb_gu)), dn(xcd_grid(a.max_tiles, nb_dn)), blk(64 * WGM * WGN),
      blkd(64 * WGM * WGND);
  hipLaunchKernelGGL((k_tiled2<TM, TN, WGM, WGN, S, SB, true, false, kMX>), gu, blk, 0, s, a, nb_gu);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (mid_event && (err = hipEventRecord(mid_event, s)) != hipSuccess) return err;
  if (a.y_dt == MOE_F32)
    hipLaunchKernelGGL((k_tiled2<TM, TND, WGM, WGND, S, SBD, false, true, kMX>), dn, blkd, 0, s, a, nb_dn);
  else
    hipLaunchKernelGGL((k_tiled2<TM, TND, WGM, WGND, S, SBD, false, false, kMX>), dn, blkd, 0, s, a, nb_dn);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_tiled(const FfnArgs& a, hipStream_t s, hipEvent_t mid_event) {
  // MXFP4: weight blocks of kMXN rows (gate/up: kMXN / 2 features) when every bank allows
  auto fits = [&](int n) {
    return a.H % n == 0 && a.bank[0].I % (n / 2) == 0 && (!a.has_shared || a.bank[1].I % (n / 2) == 0);
  };
  if (a.wdt != MOE_MXFP4 && a.tile_m == kTiledMB)
    return launch_tiled_pair<4, 4, 4, 4, 2, MOE_T2B_STAGES_B_GU, MOE_T2B_STAGES_B_DN, false>(
        a, s, mid_event);
  if (a.wdt != MOE_MXFP4)
    return launch_tiled_pair<MOE_T2_TM, MOE_T2_TN, MOE_T2_WGM, MOE_T2_WGN, MOE_T2_STAGES,
                             MOE_T2_STAGES_B_GU, MOE_T2_STAGES_B_DN, false>(a, s, mid_event);
  // MXFP4 down on 8 wavefronts of 64 x 64 (two workgroups a CU, four wavefronts a SIMD):
  // ep32_mxfp4 down 0.464 -> 0.451 ms; the same tiles for gate/up measured slower (0.905
  // -> 0.950 ms), which keeps 4 wavefronts of 64 x 128
  if (kMXN != kT2N && fits(kMXN))
    return launch_tiled_pair<MOE_T2_TM, MOE_T2_MX_TN, MOE_T2_WGM, MOE_T2_WGN, MOE_T2_MX_STAGES,
                             MOE_T2_MX_STAGES, MOE_T2_MX_STAGES, true, MOE_T2_MX_TN / 2,
                             MOE_T2_WGN * 2>(a, s, mid_event);
  return launch_tiled_pair<MOE_T2_TM, MOE_T2_TN, MOE_T2_WGM, MOE_T2_WGN, MOE_T2_MX_STAGES,
                           MOE_T2_MX_STAGES, MOE_T2_MX_STAGES, true>(a, s, mid_event);
}

}  // namespace moe
