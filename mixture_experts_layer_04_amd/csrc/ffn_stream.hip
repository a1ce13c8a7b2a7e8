// Streaming grouped-FFN kernels (few rows per expert, e.g. decode), which are bound by
// streaming the weights of the touched experts ("GC-MoE: Overlapping Expert-Parallel
// Token Dispatch with FP8/FP4 Grouped GEMM via CUDA Green Contexts", why_it_matters).
// The weights are the MFMA A operand (16 output features per wavefront), the <= 16 rows
// of the tile the B operand. Weights go straight from HBM into registers: a weight element
// is read exactly once per tile and never staged in LDS. bf16 uses
// v_mfma_f32_16x16x32_bf16, fp32 v_mfma_f32_16x16x4_f32. Because a dot product may be
// summed in any order, the K index that a lane group and register slot carry is chosen
// per kernel -- the same map for A and B -- to suit the loads: the bf16 kernels load whole
// 128-B lines of 8 rows per instruction and rearrange them across lanes (load_w_lines),
// the fp32 ones load 32 contiguous bytes of a row per lane (k0 + 8 kq + j).
// The four wavefronts of a workgroup share one block of weight rows (bf16: 4 groups of
// 16), each streaming a quarter of its K range; their fp32 partial sums meet in LDS and are
// added in K order. On r1_decode's shapes this beat halves (1%) and whole rows, and beat
// staging the down launch's h rows in LDS (0.747 against 0.769 ms).
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
#ifndef MOE_STREAM_XCD_CHUNKS  // items dealt to the XCDs in contiguous chunks
#define MOE_STREAM_XCD_CHUNKS 1
#endif

// This workgroup's (tile, feature block): XCD-chunked (xcd_chunked_item), so that the
// workgroups streaming the weights of one tile's rows share its activation rows in one L2
// (r1_decode gate/up 1.288 -> 1.262 ms, step 2.048 -> 2.021 ms; r1_decode_mxfp4 unchanged),
// or tile-major.
__device__ __forceinline__ bool stream_item(const FfnArgs& a, int fb_per_tile, int* fb, Tile* tl) {
  if (MOE_STREAM_XCD_CHUNKS) return xcd_chunked_item(a, fb_per_tile, fb, tl);
  const int tile_id = blockIdx.x / fb_per_tile;
  if (tile_id >= *a.ntiles) return false;
  *fb = blockIdx.x - tile_id * fb_per_tile;
  *tl = a.tiles[tile_id];
  return true;
}
// Workgroups of a streaming launch over max_tiles tiles of fb_per_tile items each.
inline int stream_grid(int max_tiles, int fb_per_tile) {
  return MOE_STREAM_XCD_CHUNKS ? xcd_grid(max_tiles, fb_per_tile) : max_tiles * fb_per_tile;
}

#ifndef MOE_STREAM_UNROLL_GU
#define MOE_STREAM_UNROLL_GU 2
#endif
#ifndef MOE_STREAM_UNROLL_GU_BF16  // the same for bf16 weights in whole lines (load_w_lines)
#define MOE_STREAM_UNROLL_GU_BF16 1
#endif
#ifndef MOE_STREAM_ROWS_GU  // 16-row weight groups per wavefront (bf16)
#define MOE_STREAM_ROWS_GU 4
#endif
#ifndef MOE_STREAM_ROWS_DN  // 16-row weight groups per wavefront (bf16 down)
#define MOE_STREAM_ROWS_DN 4
#endif
#ifndef MOE_STREAM_ROWS_DN_WIDE  // the same where H is a multiple of 16 of them: a
#define MOE_STREAM_ROWS_DN_WIDE 8  // workgroup's h rows then serve twice the weight rows
#endif
#ifndef MOE_STREAM_UNROLL_DN
#define MOE_STREAM_UNROLL_DN 8
#endif
#ifndef MOE_STREAM_UNROLL_DN_LINES  // K steps per iteration of the bf16 down kernel
#define MOE_STREAM_UNROLL_DN_LINES 1
#endif
#ifndef MOE_STREAM_CACHED_MULTI  // weights of groups of several tiles read through the cache
#define MOE_STREAM_CACHED_MULTI 1
#endif
#ifndef MOE_STREAM_KSPLIT_GU  // gate/up: wavefronts that share one row group, each a K range
#define MOE_STREAM_KSPLIT_GU 4
#endif
#ifndef MOE_STREAM_KSPLIT_DN  // the same for down
#define MOE_STREAM_KSPLIT_DN 4
#endif
// A wavefront's 16 R output features start at a multiple of 16 R, and ffn_shape_ok admits
// bf16 / fp32 banks with H and I multiples of 64: so 16 R must divide 64, or the last
// wavefront of an expert would read weight rows of the next expert (past the last one's
// end) and write h or y past the row's end.
static_assert(64 % (16 * MOE_STREAM_ROWS_GU) == 0, "gate/up row groups must tile I % 64");
static_assert(64 % (16 * MOE_STREAM_ROWS_DN) == 0, "down row groups must tile H % 64");
// (the wide down variant is launched only where 16 MOE_STREAM_ROWS_DN_WIDE divides H)
// Weight fragment: ordinary cached loads (on MI355X they measured faster than
// non-temporal ones for this many-rows-at-once pattern).
__device__ __forceinline__ Frag32 load_w(const void* p) { return load_c(p); }

// bf16 weight rows in whole 128-B lines. A load instruction whose 64 lanes take 16 rows x
// 64 B (lane (m, kq) its MFMA fragment) streamed at 5.5 TB/s non-temporal and 6.2 TB/s
// cached in a probe on MI355X; one whose lanes take 8 rows x 128 B streamed at 6.7-6.8
// TB/s non-temporal. So a 16-row group's 64-element K step (16 rows x 128 B) is two such
// loads, G0 (rows 0..7) and G1 (rows 8..15): lane (m, kq) takes 16-B chunk kq + 4 (m / 8)
// of row m % 8 in G0 and chunk kq + 4 (1 - m / 8) of row 8 + m % 8 in G1. Then row m's
// chunk kq sits in lane (m, kq) of G0 (m < 8) or G1 (m >= 8), and its chunk kq + 4 in lane
// (m ^ 8, kq) of the other one: a select and a DPP rotation by 8 lanes within each row of
// 16 give the MFMA operand, .lo = K elements 8 kq .. 8 kq + 7 and .hi = 32 + 8 kq .. of
// the step. The B operand takes the same K map (load_x_perm).
struct WRaw {
  u32x4 g0, g1;
};
struct WLane {  // this lane's byte offsets of G0 and G1 from a group's first row
  uint32_t o0, o1;
  bool lo8;
};
__device__ __forceinline__ WLane wlane(int m, int kq, uint32_t row_bytes) {
  return WLane{(uint32_t)(m & 7) * row_bytes + (uint32_t)(kq + 4 * (m >> 3)) * 16,
               (uint32_t)(8 + (m & 7)) * row_bytes + (uint32_t)(kq + 4 * (1 - (m >> 3))) * 16, m < 8};
}
// kNT: with the non-temporal hint (weights read once); without it for groups of more than
// one tile, whose tiles read the same weights and share them only through the cache.
template <bool kNT = true>
__device__ __forceinline__ WRaw load_w_lines(const char* group, const WLane& w) {
  WRaw r;
  if constexpr (kNT) {
    r.g0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(group + w.o0));
    r.g1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(group + w.o1));
  } else {
    r.g0 = *reinterpret_cast<const u32x4*>(group + w.o0);
    r.g1 = *reinterpret_cast<const u32x4*>(group + w.o1);
  }
  return r;
}
__device__ __forceinline__ Frag32 w_frag(const WRaw& r, bool lo8) {
  Frag32 f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f.lo[j] = lo8 ? r.g0[j] : r.g1[j];
    const uint32_t y = lo8 ? r.g1[j] : r.g0[j];
    // row_ror:8 -- lane i of each 16-lane row takes lane (i + 8) % 16
    f.hi[j] = (uint32_t)__builtin_amdgcn_mov_dpp((int)y, 0x128, 0xF, 0xF, false);
  }
  return f;
}
// The matching B-operand fragment of a row: K elements 8 kq .. + 7 and 32 + 8 kq .. + 7 of
// the step (p already offset by 16 kq bytes); zeros for padding rows.
__device__ __forceinline__ Frag32 load_x_perm(const char* p, bool valid) {
  Frag32 f;
  if (valid) {
    f.lo = *reinterpret_cast<const u32x4*>(p);
    f.hi = *reinterpret_cast<const u32x4*>(p + 64);
  } else {
    f.lo = u32x4{0, 0, 0, 0};
    f.hi = u32x4{0, 0, 0, 0};
  }
  return f;
}
// Activation fragment of a row; lanes of padding rows (beyond the tile's rows) load
// nothing and contribute zeros to columns that are never stored.
__device__ __forceinline__ Frag32 load_x(const void* p, bool valid) {
  if (valid) return load_c(p);
  Frag32 z;
  z.lo = u32x4{0, 0, 0, 0};
  z.hi = u32x4{0, 0, 0, 0};
  return z;
}

// h's residual for K step k0 (64 elements) of the bf16 down projection, in load_w_lines' K
// map: elements k0 + 8 kq .. + 7 (.lo) and k0 + 32 + 8 kq .. + 7 (.hi), i.e. the code words
// 4 kq and 16 + 4 kq bytes into the step (lr already offset by 4 kq), decoded with the
// E8M0 scales of the step's two 32-element blocks; zeros for padding rows.
__device__ __forceinline__ Frag32 load_lo_perm(const uint8_t* lr, const uint8_t* ls, int k0,
                                               bool valid) {
  Frag32 f;
  if (!valid) {
    f.lo = u32x4{0, 0, 0, 0};
    f.hi = u32x4{0, 0, 0, 0};
    return f;
  }
  const uint32_t q0 = *reinterpret_cast<const uint32_t*>(lr + k0 / 2);
  const uint32_t q1 = *reinterpret_cast<const uint32_t*>(lr + k0 / 2 + 16);
  const uint32_t sc = *reinterpret_cast<const uint16_t*>(ls + k0 / 32);
  f.lo = __builtin_bit_cast(u32x4, e2m1x8_bf16(q0, e8m0_f32_fast(sc & 0xFFu)));
  f.hi = __builtin_bit_cast(u32x4, e2m1x8_bf16(q1, e8m0_f32_fast(sc >> 8)));
  return f;
}

template <bool kF32>
__device__ __forceinline__ f32x4 mma(const Frag32& w, const Frag32& x, f32x4 acc) {
  return kF32 ? mma_f32(w, x, acc) : mma_bf16(w, x, acc);
}

// Gate/up + SwiGLU. Workgroup = (tile, block of 64 R / KS h features); wavefronts
// w = KS q + ks compute features [f0, f0 + 16 R) of h, f0 from q, over K range ks: gate
// rows f0.. and up rows I + f0.. of W13[e], R groups of 16 rows each reusing one
// activation fragment per K step.
template <bool kF32, int R>
__global__ void __launch_bounds__(256) k_gateup_stream(FfnArgs a, int fb_per_tile) {
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  int fb;
  Tile tl;
  if (!stream_item(a, fb_per_tile, &fb, &tl)) return;
  const int bank = tl.group < a.E ? 0 : 1;
  const int64_t ge = tl.group < a.E ? tl.group : 0;
  const int I = a.bank[bank].I;
  const int H = a.H;
  constexpr int KS = MOE_STREAM_KSPLIT_GU;
  static_assert(4 % KS == 0, "K split divides the workgroup");
  const int ks = wave % KS;
  const int f0 = (fb * (4 / KS) + wave / KS) * 16 * R;
  if (KS == 1 && f0 >= I) return;
  const bool active = f0 < I;
  const int m = l & 15, kq = l >> 4;
  const int esz = kF32 ? 4 : 2;
  const char* w13 = reinterpret_cast<const char*>(a.bank[bank].w13) + ge * 2 * I * (int64_t)H * esz;
  const bool xv = m < tl.nrows;
  const int row = tl.row0 + (xv ? m : 0);
  const int64_t src = a.a_rowmap ? a.a_rowmap[row] : row;
  constexpr int kStep = kF32 ? 32 : 64;          // K elements per MFMA step
  constexpr int kLane = kStep / 4;               // contiguous elements per lane per step
  constexpr int U = MOE_STREAM_UNROLL_GU;
  f32x4 accg[R], accu[R];
#pragma unroll
  for (int r = 0; r < R; ++r) accg[r] = accu[r] = f32x4{0, 0, 0, 0};
  const int nst = H / kStep;
  const int kbeg = active ? (ks * nst / KS) * kStep : 0;
  const int kend = active ? ((ks + 1) * nst / KS) * kStep : 0;
  const int kmain = kend - (kend - kbeg) % (kStep * U);
  if constexpr (!kF32) {
    // whole 128-B lines of 8 rows per load (load_w_lines): the group's first row is uniform
    const WLane wl = wlane(m, kq, (uint32_t)H * 2);
    const char* xq = reinterpret_cast<const char*>(a.a) + src * H * 2 + kq * 16;
    const char* g0 = w13 + (int64_t)f0 * H * 2;
    const char* u0 = w13 + (int64_t)(I + f0) * H * 2;
    auto step = [&](int k0, auto uc, auto ntc) {
      constexpr int UU = decltype(uc)::value;
      constexpr bool NT = decltype(ntc)::value != 0;
      WRaw rg[UU][R], ru[UU][R];
      Frag32 fx[UU];
#pragma unroll
      for (int u = 0; u < UU; ++u) {
        const int64_t o = (int64_t)(k0 + u * 64) * 2;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          rg[u][r] = load_w_lines<NT>(g0 + (int64_t)16 * r * H * 2 + o, wl);
          ru[u][r] = load_w_lines<NT>(u0 + (int64_t)16 * r * H * 2 + o, wl);
        }
        fx[u] = load_x_perm(xq + o, xv);
      }
#pragma unroll
      for (int u = 0; u < UU; ++u)
#pragma unroll
        for (int r = 0; r < R; ++r) {
          accg[r] = mma_bf16(w_frag(rg[u][r], wl.lo8), fx[u], accg[r]);
          accu[r] = mma_bf16(w_frag(ru[u][r], wl.lo8), fx[u], accu[r]);
        }
    };
    constexpr int UB = MOE_STREAM_UNROLL_GU_BF16;
    const int kmb = kend - (kend - kbeg) % (64 * UB);
    // a group of one tile streams its weights past the cache; the tiles of a larger group
    // (a hot expert, the shared expert) read them through it, where they meet: with the
    // hint on every group the second tile of each 17-32-row expert fetched the weights
    // again (r1_decode gate/up 1.328 -> 1.291 ms, down 0.726 -> 0.708 ms)
    auto kloop = [&](auto ntc) {
      for (int k0 = kbeg; k0 < kmb; k0 += 64 * UB) step(k0, IntC<UB>{}, ntc);
      for (int k0 = kmb; k0 < kend; k0 += 64) step(k0, IntC<1>{}, ntc);
    };
    if (!MOE_STREAM_CACHED_MULTI || tl.nblk == 1) kloop(IntC<1>{});
    else kloop(IntC<0>{});
  } else {
    // fp32: each lane's 32 contiguous bytes of its row per step (cached loads), K index
    // k0 + 8 kq + j in both operands
    const int64_t lane_off = (int64_t)kq * kLane * esz;
    const char* wg[R];
    const char* wu[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      wg[r] = w13 + (int64_t)(f0 + 16 * r + m) * H * esz + lane_off;
      wu[r] = w13 + (int64_t)(I + f0 + 16 * r + m) * H * esz + lane_off;
    }
    const char* xr = reinterpret_cast<const char*>(a.a) + src * H * esz + lane_off;
    for (int k0 = kbeg; k0 < kmain; k0 += kStep * U) {
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
    for (int k0 = kmain; k0 < kend; k0 += kStep) {
      const int64_t o = (int64_t)k0 * esz;
      const Frag32 fx = load_x(xr + o, xv);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        accg[r] = mma<kF32>(load_w(wg[r] + o), fx, accg[r]);
        accu[r] = mma<kF32>(load_w(wu[r] + o), fx, accu[r]);
      }
    }
  }
  if constexpr (KS > 1) {
    // the K ranges' partial sums meet in LDS; the first wavefront of each row group adds
    // them in K order
    __shared__ f32x4 red[4][2 * R][64];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      red[wave][r][l] = accg[r];
      red[wave][R + r][l] = accu[r];
    }
    __syncthreads();
    if (ks != 0 || !active) return;
#pragma unroll
    for (int j = 1; j < KS; ++j)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const f32x4 g = red[wave + j][r][l], u = red[wave + j][R + r][l];
        accg[r] = f32x4{accg[r][0] + g[0], accg[r][1] + g[1], accg[r][2] + g[2], accg[r][3] + g[3]};
        accu[r] = f32x4{accu[r][0] + u[0], accu[r][1] + u[1], accu[r][2] + u[2], accu[r][3] + u[3]};
      }
  }
  if (!xv) return;
  if constexpr (kF32) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      f32x4 hv;
#pragma unroll
      for (int i = 0; i < 4; ++i) hv[i] = silu_mul(accg[r][i], accu[r][i]);
      store4<true>(a.h, (int64_t)(tl.row0 + m) * a.I_max + f0 + 16 * r + kq * 4, hv);
    }
  } else {
    // h = hi + lo (ffn_common.h): row groups 2 j and 2 j + 1 make one 32-feature block,
    // whose 32 values sit in this lane (8) and the lanes of the other kq (same m)
    static_assert(R % 2 == 0, "32-feature blocks of the residual");
    const int64_t row = tl.row0 + m;
#pragma unroll
    for (int r2 = 0; r2 < R; r2 += 2) {
      float lo[2][4];
      float am = 0.0f;
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        uint2 p;
        uint16_t b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          b[i] = split_bf16(silu_mul(accg[r2 + d][i], accu[r2 + d][i]), &lo[d][i]);
          am = fmaxf(am, fabsf(lo[d][i]));
        }
        p.x = (uint32_t)b[0] | ((uint32_t)b[1] << 16);
        p.y = (uint32_t)b[2] | ((uint32_t)b[3] << 16);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.h) + row * a.I_max + f0 +
                                  16 * (r2 + d) + kq * 4) = p;
      }
      am = fmaxf(am, __shfl_xor(am, 16, 64));
      am = fmaxf(am, __shfl_xor(am, 32, 64));
      const int e = mx_exponent(am);
      const float inv = exp2i(-e);
      const int fblk = f0 + 16 * r2;  // first feature of the block
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        // features 16 d + 4 kq .. + 3 of the block: bytes 8 d + 2 kq, 8 d + 2 kq + 1
        const uint32_t c0 = e2m1_code(lo[d][0] * inv), c1 = e2m1_code(lo[d][1] * inv);
        const uint32_t c2 = e2m1_code(lo[d][2] * inv), c3 = e2m1_code(lo[d][3] * inv);
        *reinterpret_cast<uint16_t*>(a.h_lo + row * (a.I_max / 2) + fblk / 2 + 8 * d + 2 * kq) =
            (uint16_t)(c0 | (c1 << 4) | (c2 << 8) | (c3 << 12));
      }
      if (kq == 0) a.h_lo_s[row * lo_sstride(a.I_max) + fblk / 32] = (uint8_t)(e + 127);
    }
  }
}

// Down projection. Workgroup = (tile, block of 64 R / KS output features of H); wavefronts
// w = KS q + ks compute R groups of 16 output features over K range ks, reusing one h
// fragment per K step.
template <bool kF32, bool kYF32, int R>
__global__ void __launch_bounds__(256) k_down_stream(FfnArgs a, int fb_per_tile) {
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  int fb;
  Tile tl;
  if (!stream_item(a, fb_per_tile, &fb, &tl)) return;
  const int bank = tl.group < a.E ? 0 : 1;
  const int64_t ge = tl.group < a.E ? tl.group : 0;
  const int I = a.bank[bank].I;
  const int H = a.H;
  constexpr int KS = MOE_STREAM_KSPLIT_DN;
  static_assert(4 % KS == 0, "K split divides the workgroup");
  const int ks = wave % KS;
  const int f0 = (fb * (4 / KS) + wave / KS) * 16 * R;
  if (KS == 1 && f0 >= H) return;
  const bool active = f0 < H;
  const int m = l & 15, kq = l >> 4;
  constexpr int kStep = kF32 ? 32 : 64;  // K elements per MFMA step
  // this wavefront's K range [kbeg, kend), whole K steps
  const int nst = I / kStep;
  const int kbeg = active ? (ks * nst / KS) * kStep : 0;
  const int kend = active ? ((ks + 1) * nst / KS) * kStep : 0;
  const bool xv = m < tl.nrows;
  const int64_t hrow = tl.row0 + (xv ? m : 0);
  f32x4 acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = f32x4{0, 0, 0, 0};
  if constexpr (!kF32) {
    // bf16: weights in whole 128-B lines (load_w_lines); h and its residual (ffn_common.h)
    // in that K map
    const char* w2 = reinterpret_cast<const char*>(a.bank[bank].w2) + ge * (int64_t)H * I * 2;
    const WLane wl = wlane(m, kq, (uint32_t)I * 2);
    const char* hq = reinterpret_cast<const char*>(a.h) + hrow * a.I_max * 2 + kq * 16;
    const uint8_t* lq = a.h_lo + hrow * (a.I_max / 2) + kq * 4;
    const uint8_t* lsb = a.h_lo_s + hrow * lo_sstride(a.I_max);
    auto step = [&](int k0, auto uc, auto ntc) {
      constexpr int UU = decltype(uc)::value;
      constexpr bool NT = decltype(ntc)::value != 0;
      WRaw rw[UU][R];
      Frag32 fh[UU], fl[UU];
#pragma unroll
      for (int u = 0; u < UU; ++u) {
        const int64_t o = (int64_t)(k0 + u * 64) * 2;
#pragma unroll
        for (int r = 0; r < R; ++r)
          rw[u][r] = load_w_lines<NT>(w2 + (int64_t)(f0 + 16 * r) * I * 2 + o, wl);
        fh[u] = load_x_perm(hq + o, xv);
        fl[u] = load_lo_perm(lq, lsb, k0 + u * 64, xv);
      }
#pragma unroll
      for (int u = 0; u < UU; ++u)
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const Frag32 fw = w_frag(rw[u][r], wl.lo8);
          acc[r] = mma_bf16(fw, fh[u], acc[r]);
          acc[r] = mma_bf16(fw, fl[u], acc[r]);
        }
    };
    constexpr int UB = MOE_STREAM_UNROLL_DN_LINES;
    const int kmb = kend - (kend - kbeg) % (64 * UB);
    auto kloop = [&](auto ntc) {  // as in the gate/up launch
      for (int k0 = kbeg; k0 < kmb; k0 += 64 * UB) step(k0, IntC<UB>{}, ntc);
      for (int k0 = kmb; k0 < kend; k0 += 64) step(k0, IntC<1>{}, ntc);
    };
    if (!MOE_STREAM_CACHED_MULTI || tl.nblk == 1) kloop(IntC<1>{});
    else kloop(IntC<0>{});
  } else {
    // fp32: each lane's 32 contiguous bytes of its row per step (cached loads), K index
    // k0 + 8 kq + j in both operands
    constexpr int U = MOE_STREAM_UNROLL_DN;
    const int64_t lane_off = (int64_t)kq * 8 * 4;
    const char* w2 = reinterpret_cast<const char*>(a.bank[bank].w2) + ge * (int64_t)H * I * 4;
    const char* wr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) wr[r] = w2 + (int64_t)(f0 + 16 * r + m) * I * 4 + lane_off;
    const char* hr = reinterpret_cast<const char*>(a.h) + hrow * a.I_max * 4 + lane_off;
    const int kmain = kend - (kend - kbeg) % (kStep * U);
    for (int k0 = kbeg; k0 < kmain; k0 += kStep * U) {
      Frag32 fw[U][R], fh[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t o = (int64_t)(k0 + u * kStep) * 4;
#pragma unroll
        for (int r = 0; r < R; ++r) fw[u][r] = load_w(wr[r] + o);
        fh[u] = load_x(hr + o, xv);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = mma_f32(fw[u][r], fh[u], acc[r]);
    }
    for (int k0 = kmain; k0 < kend; k0 += kStep) {
      const int64_t o = (int64_t)k0 * 4;
      const Frag32 fh = load_x(hr + o, xv);
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = mma_f32(load_w(wr[r] + o), fh, acc[r]);
    }
  }
  if constexpr (KS > 1) {
    // the K ranges' partial sums meet in LDS; the first wavefront of each row group adds
    // them in K order and stores
    __shared__ f32x4 red[4][R][64];
#pragma unroll
    for (int r = 0; r < R; ++r) red[wave][r][l] = acc[r];
    __syncthreads();
    if (ks != 0 || !active) return;
#pragma unroll
    for (int j = 1; j < KS; ++j)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const f32x4 v = red[wave + j][r][l];
        acc[r] = f32x4{acc[r][0] + v[0], acc[r][1] + v[1], acc[r][2] + v[2], acc[r][3] + v[3]};
      }
  }
  if (xv) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      store4<kYF32>(a.y, (int64_t)(tl.row0 + m) * H + f0 + 16 * r + kq * 4, acc[r]);
  }
}

// ------------------------------------------------------------------ MXFP4 weights
// The same streaming scheme for MXFP4 weights (E2M1 codes, 2 a byte, with an E8M0 scale
// per 32 elements). An iteration covers 256 U elements of every weight row: 128 U bytes of
// codes, read as 2 U loads of 64 contiguous bytes a row (16 B for each of the 4 lane
// groups kq: load i gives lane group kq the 32 elements from 32 kq + 128 i), plus the
// 8 U scale bytes of those elements (all lanes of a row load them; lane group kq uses
// byte kq of each dword). Word w of a lane's codes is decoded exactly to bf16 in registers
// and multiplied with the same 8 elements of the activation row by one
// v_mfma_f32_16x16x32_bf16, so a (lane group, word) pair carries the same K index in both
// operands.
#ifndef MOE_STREAM_MX_U
#define MOE_STREAM_MX_U 2
#endif
#ifndef MOE_STREAM_MX_LDS  // activation rows staged in LDS, shared by the workgroup
#define MOE_STREAM_MX_LDS 1
#endif
#ifndef MOE_STREAM_MX_ROWS_GU
#define MOE_STREAM_MX_ROWS_GU 1
#endif
#ifndef MOE_STREAM_MX_LINES  // MXFP4 codes in whole 128-B lines (load_mx_lines)
#define MOE_STREAM_MX_LINES 1
#endif
#ifndef MOE_STREAM_MX_ROWS_DN
#define MOE_STREAM_MX_ROWS_DN 4
#endif
constexpr int kMxStreamK = 256 * MOE_STREAM_MX_U;  // K elements per iteration (divides H, I)
// The wavefronts' 16 R-row groups must tile H and I exactly (both multiples of kMxStreamK):
// a partial group would read weight rows past its expert's.
static_assert(kMxStreamK % (16 * MOE_STREAM_MX_ROWS_GU) == 0 &&
                  kMxStreamK % (16 * MOE_STREAM_MX_ROWS_DN) == 0,
              "MXFP4 streaming row groups must divide the K iteration");

template <int U>
struct MxCodes {  // this lane's 32 U bytes of E2M1 codes and the row's 8 U scale bytes
  u32x4 q[2 * U];
  uint32_t sc[2 * U];
};

// codes: the row's codes at the iteration's start, already offset by 16 kq; scales: the
// row's scale bytes at the iteration's start
template <int U>
__device__ __forceinline__ MxCodes<U> load_mx(const uint8_t* codes, const uint8_t* scales) {
  MxCodes<U> c;
#pragma unroll
  for (int i = 0; i < 2 * U; ++i) c.q[i] = *reinterpret_cast<const u32x4*>(codes + 64 * i);
  if (U == 2) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(scales);
#pragma unroll
    for (int i = 0; i < 2 * U; ++i) c.sc[i] = v[i];
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(scales);
    c.sc[0] = v.x;
    c.sc[1 % (2 * U)] = v.y;
  }
  return c;
}

// acc += (decoded codes) x (8 U bf16x8 activation fragments); kq: this lane's group
template <int U>
__device__ __forceinline__ f32x4 mma_mx(const MxCodes<U>& w, const u32x4* x, int kq, f32x4 acc) {
#pragma unroll
  for (int i = 0; i < 2 * U; ++i) {
    const float sc = e8m0_f32((w.sc[i] >> (8 * kq)) & 0xFFu);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 a = e2m1x8_bf16(w.q[i][j], sc);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(x[4 * i + j]), acc, 0, 0, 0);
    }
  }
  return acc;
}

// the activation elements that match a lane's codes: 32 from 32 kq + 128 i for each i
// (p: the row at the iteration's start, already offset by 64 kq bytes)
template <int U>
__device__ __forceinline__ void load_x_mx(const char* p, bool valid, u32x4* x) {
#pragma unroll
  for (int i = 0; i < 2 * U; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      x[4 * i + j] = valid ? *reinterpret_cast<const u32x4*>(p + 256 * i + 16 * j) : u32x4{0, 0, 0, 0};
}

// Activation rows staged in LDS (U == 2): an iteration's 512 elements of the tile's 16
// rows (1 KB a row, 16 KB a chunk) go global -> LDS by DMA through two buffers shared by
// the workgroup's four wavefronts; wavefront w stages rows 4 w .. 4 w + 3, lane l of row
// p taking the row's 16-B piece l ^ p. Lane (m, kq) then reads pieces 4 kq + 16 i + j of
// row m, the ones load_x_mx reads from global memory.
constexpr int kMxChunk = 16 * 1024;
// The four pieces of word group i (read just before use, so that only 16 registers
// hold activations).
__device__ __forceinline__ void read_x_mx_lds(const char* buf, int m, int kq, int i, u32x4* x4) {
  const char* rb = buf + m * 1024;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    x4[j] = *reinterpret_cast<const u32x4*>(rb + (((4 * kq + 16 * i + j) ^ m) << 4));
}
// The same codes in whole 128-B lines (load_w_lines, non-temporal): line pair p of a
// 16-row group and iteration covers the row's bytes 128 p .. 128 p + 127, whose chunk kq
// (elements 256 p + 32 kq ..) is this lane's word group 2 p and chunk kq + 4 (elements
// 256 p + 128 + 32 kq ..) its word group 2 p + 1 -- the K map of load_mx. The lines stay
// as loaded until a word group is used (mx_words), so that the loads stay in flight.
template <int U>
struct MxLines {
  WRaw p[U];
  uint32_t sc[2 * U];
};
// grp: the group's first row's codes at the iteration's start; scales: this lane's row's
// (Reading the codes of groups of several tiles through the cache, as the bf16 kernels do,
// measured slower here: r1_decode_mxfp4 gate/up 0.425 -> 0.454 ms.)
template <int U>
__device__ __forceinline__ MxLines<U> load_mx_lines(const uint8_t* grp, const WLane& wl,
                                                    const uint8_t* scales) {
  MxLines<U> c;
#pragma unroll
  for (int p = 0; p < U; ++p) c.p[p] = load_w_lines(reinterpret_cast<const char*>(grp) + 128 * p, wl);
  if (U == 2) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(scales);
#pragma unroll
    for (int i = 0; i < 2 * U; ++i) c.sc[i] = v[i];
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(scales);
    c.sc[0] = v.x;
    c.sc[1 % (2 * U)] = v.y;
  }
  return c;
}
// word group i of the lines, as load_mx would hold it
template <int U>
__device__ __forceinline__ u32x4 mx_words(const MxLines<U>& w, int i, bool lo8) {
  const WRaw& r = w.p[i >> 1];
  u32x4 q;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if ((i & 1) == 0) {
      q[j] = lo8 ? r.g0[j] : r.g1[j];
    } else {
      const uint32_t y = lo8 ? r.g1[j] : r.g0[j];
      q[j] = (uint32_t)__builtin_amdgcn_mov_dpp((int)y, 0x128, 0xF, 0xF, false);  // row_ror:8
    }
  }
  return q;
}
template <int U>
__device__ __forceinline__ f32x4 mma_mx_part(const MxLines<U>& w, bool lo8, const u32x4* x4, int i,
                                             int kq, f32x4 acc) {
  const float sc = e8m0_f32((w.sc[i] >> (8 * kq)) & 0xFFu);
  const u32x4 q = mx_words<U>(w, i, lo8);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e2m1x8_bf16(q[j], sc), as_bf16x8(x4[j]), acc,
                                                  0, 0, 0);
  return acc;
}

// acc += word group i of w (decoded with its scale) x the matching 4 activation pieces
template <int U>
__device__ __forceinline__ f32x4 mma_mx_part(const MxCodes<U>& w, const u32x4* x4, int i, int kq,
                                             f32x4 acc) {
  const float sc = e8m0_f32((w.sc[i] >> (8 * kq)) & 0xFFu);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e2m1x8_bf16(w.q[i][j], sc), as_bf16x8(x4[j]), acc,
                                                  0, 0, 0);
  return acc;
}

// Gate/up + SwiGLU: wavefront w computes features [f0, f0 + 16 R) of h from the gate rows
// f0.. and the up rows I + f0.. of W13[e].
template <int R, int U>
__global__ void __launch_bounds__(256) k_gateup_stream_mx(FfnArgs a, int fb_per_tile) {
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  int fb;
  Tile tl;
  if (!stream_item(a, fb_per_tile, &fb, &tl)) return;
  const int bank = tl.group < a.E ? 0 : 1;
  const int64_t ge = tl.group < a.E ? tl.group : 0;
  const int I = a.bank[bank].I;
  const int H = a.H;
  const int f0 = (fb * 4 + wave) * 16 * R;
  if (!MOE_STREAM_MX_LDS && f0 >= I) return;
  const bool active = f0 < I;
  const int m = l & 15, kq = l >> 4;
  const uint8_t* codes = reinterpret_cast<const uint8_t*>(a.bank[bank].w13) + ge * 2 * I * (int64_t)(H / 2);
  const uint8_t* scales = reinterpret_cast<const uint8_t*>(a.bank[bank].w13_scale) + ge * 2 * I * (int64_t)(H / 32);
  const uint8_t *cg[R], *cu[R], *sg[R], *su[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t g = (active ? f0 : 0) + 16 * r + m, u = I + g;
    cg[r] = codes + g * (H / 2) + 16 * kq;
    cu[r] = codes + u * (H / 2) + 16 * kq;
    sg[r] = scales + g * (H / 32);
    su[r] = scales + u * (H / 32);
  }
  const bool xv = m < tl.nrows;
#if !MOE_STREAM_MX_LDS
  const int row = tl.row0 + (xv ? m : 0);
  const int64_t src = a.a_rowmap ? a.a_rowmap[row] : row;
  const char* xr = reinterpret_cast<const char*>(a.a) + src * H * 2 + 64 * kq;
#endif
  f32x4 accg[R], accu[R];
#pragma unroll
  for (int r = 0; r < R; ++r) accg[r] = accu[r] = f32x4{0, 0, 0, 0};
#if MOE_STREAM_MX_LDS
  static_assert(U == 2, "LDS staging of 1-KB row pieces");
  __shared__ __attribute__((aligned(1024))) char xs[2 * kMxChunk];
  const char* xsrc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p = 4 * wave + j;
    const int rp = tl.row0 + (p < tl.nrows ? p : (tl.nrows > 0 ? tl.nrows - 1 : 0));
    const int64_t sp = a.a_rowmap ? a.a_rowmap[rp] : rp;
    xsrc[j] = reinterpret_cast<const char*>(a.a) + sp * H * 2 + (l ^ p) * 16;
  }
  auto issue = [&](int c) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dma16(xsrc[j] + (int64_t)c * 1024, xs + (c & 1) * kMxChunk + (4 * wave + j) * 1024);
  };
  issue(0);
#endif
#if MOE_STREAM_MX_LDS && MOE_STREAM_MX_LINES
  const WLane wl = wlane(m, kq, (uint32_t)(H / 2));
  const uint8_t* glg = codes + (int64_t)(active ? f0 : 0) * (H / 2);
  const uint8_t* glu = codes + (int64_t)(I + (active ? f0 : 0)) * (H / 2);
#endif
  for (int k0 = 0, c = 0; k0 < H; k0 += 256 * U, ++c) {
#if MOE_STREAM_MX_LDS && MOE_STREAM_MX_LINES
    MxLines<U> wg[R], wu[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      wg[r] = load_mx_lines<U>(glg + (int64_t)16 * r * (H / 2) + k0 / 2, wl, sg[r] + k0 / 32);
      wu[r] = load_mx_lines<U>(glu + (int64_t)16 * r * (H / 2) + k0 / 2, wl, su[r] + k0 / 32);
    }
#else
    MxCodes<U> wg[R], wu[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      wg[r] = load_mx<U>(cg[r] + k0 / 2, sg[r] + k0 / 32);
      wu[r] = load_mx<U>(cu[r] + k0 / 2, su[r] + k0 / 32);
    }
#endif
#if MOE_STREAM_MX_LDS
    wait_vmcnt<2 * R * (2 * U + 1)>();  // this wavefront's DMA of chunk c (before the weight loads)
    __builtin_amdgcn_s_barrier();       // ... and the others'; chunk c - 1 is read
    if (k0 + 256 * U < H) issue(c + 1);
#pragma unroll
    for (int i = 0; i < 2 * U; ++i) {
      u32x4 x4[4];
      read_x_mx_lds(xs + (c & 1) * kMxChunk, m, kq, i, x4);
#pragma unroll
      for (int r = 0; r < R; ++r) {
#if MOE_STREAM_MX_LINES
        accg[r] = mma_mx_part<U>(wg[r], wl.lo8, x4, i, kq, accg[r]);
        accu[r] = mma_mx_part<U>(wu[r], wl.lo8, x4, i, kq, accu[r]);
#else
        accg[r] = mma_mx_part<U>(wg[r], x4, i, kq, accg[r]);
        accu[r] = mma_mx_part<U>(wu[r], x4, i, kq, accu[r]);
#endif
      }
    }
#else
    u32x4 x[8 * U];
    load_x_mx<U>(xr + (int64_t)k0 * 2, xv, x);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      accg[r] = mma_mx<U>(wg[r], x, kq, accg[r]);
      accu[r] = mma_mx<U>(wu[r], x, kq, accu[r]);
    }
#endif
  }
  if (xv && active) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      f32x4 hv;
#pragma unroll
      for (int i = 0; i < 4; ++i) hv[i] = silu_mul(accg[r][i], accu[r][i]);
      store4<false>(a.h, (int64_t)(tl.row0 + m) * a.I_max + f0 + 16 * r + kq * 4, hv);
    }
  }
}

// Down projection: wavefront w computes output features [f0, f0 + 16 R) from W2[e] rows.
template <bool kYF32, int R, int U>
__global__ void __launch_bounds__(256) k_down_stream_mx(FfnArgs a, int fb_per_tile) {
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  int fb;
  Tile tl;
  if (!stream_item(a, fb_per_tile, &fb, &tl)) return;
  const int bank = tl.group < a.E ? 0 : 1;
  const int64_t ge = tl.group < a.E ? tl.group : 0;
  const int I = a.bank[bank].I;
  const int H = a.H;
  const int f0 = (fb * 4 + wave) * 16 * R;
  if (!MOE_STREAM_MX_LDS && f0 >= H) return;
  const bool active = f0 < H;
  const int m = l & 15, kq = l >> 4;
  const uint8_t* codes = reinterpret_cast<const uint8_t*>(a.bank[bank].w2) + ge * (int64_t)H * (I / 2);
  const uint8_t* scales = reinterpret_cast<const uint8_t*>(a.bank[bank].w2_scale) + ge * (int64_t)H * (I / 32);
  const uint8_t *cw[R], *sw[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t o = (active ? f0 : 0) + 16 * r + m;
    cw[r] = codes + o * (I / 2) + 16 * kq;
    sw[r] = scales + o * (I / 32);
  }
  const bool xv = m < tl.nrows;
#if !MOE_STREAM_MX_LDS
  const char* hr = reinterpret_cast<const char*>(a.h) +
                   (int64_t)(tl.row0 + (xv ? m : 0)) * a.I_max * 2 + 64 * kq;
#endif
  f32x4 acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = f32x4{0, 0, 0, 0};
#if MOE_STREAM_MX_LDS
  static_assert(U == 2, "LDS staging of 1-KB row pieces");
  __shared__ __attribute__((aligned(1024))) char xs[2 * kMxChunk];
  const char* xsrc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p = 4 * wave + j;
    const int rp = tl.row0 + (p < tl.nrows ? p : (tl.nrows > 0 ? tl.nrows - 1 : 0));
    xsrc[j] = reinterpret_cast<const char*>(a.h) + (int64_t)rp * a.I_max * 2 + (l ^ p) * 16;
  }
  auto issue = [&](int c) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dma16(xsrc[j] + (int64_t)c * 1024, xs + (c & 1) * kMxChunk + (4 * wave + j) * 1024);
  };
  issue(0);
#endif
#if MOE_STREAM_MX_LDS && MOE_STREAM_MX_LINES
  const WLane wl = wlane(m, kq, (uint32_t)(I / 2));
  const uint8_t* gl = codes + (int64_t)(active ? f0 : 0) * (I / 2);
#endif
  for (int k0 = 0, c = 0; k0 < I; k0 += 256 * U, ++c) {
#if MOE_STREAM_MX_LDS && MOE_STREAM_MX_LINES
    MxLines<U> w[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
      w[r] = load_mx_lines<U>(gl + (int64_t)16 * r * (I / 2) + k0 / 2, wl, sw[r] + k0 / 32);
#else
    MxCodes<U> w[R];
#pragma unroll
    for (int r = 0; r < R; ++r) w[r] = load_mx<U>(cw[r] + k0 / 2, sw[r] + k0 / 32);
#endif
#if MOE_STREAM_MX_LDS
    wait_vmcnt<R * (2 * U + 1)>();
    __builtin_amdgcn_s_barrier();
    if (k0 + 256 * U < I) issue(c + 1);
#pragma unroll
    for (int i = 0; i < 2 * U; ++i) {
      u32x4 x4[4];
      read_x_mx_lds(xs + (c & 1) * kMxChunk, m, kq, i, x4);
#pragma unroll
      for (int r = 0; r < R; ++r) {
#if MOE_STREAM_MX_LINES
        acc[r] = mma_mx_part<U>(w[r], wl.lo8, x4, i, kq, acc[r]);
#else
        acc[r] = mma_mx_part<U>(w[r], x4, i, kq, acc[r]);
#endif
      }
    }
#else
    u32x4 x[8 * U];
    load_x_mx<U>(hr + (int64_t)k0 * 2, xv, x);
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = mma_mx<U>(w[r], x, kq, acc[r]);
#endif
  }
  if (xv && active) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      store4<kYF32>(a.y, (int64_t)(tl.row0 + m) * H + f0 + 16 * r + kq * 4, acc[r]);
  }
}

}  // namespace

bool ffn_stream_mx_ok(int32_t H, int32_t I) { return H % kMxStreamK == 0 && I % kMxStreamK == 0; }

hipError_t launch_ffn_stream(const FfnArgs& a, hipStream_t s, hipEvent_t mid_event) {
  constexpr int RG = MOE_STREAM_ROWS_GU, RD = MOE_STREAM_ROWS_DN, RDW = MOE_STREAM_ROWS_DN_WIDE;
  constexpr int KSG = MOE_STREAM_KSPLIT_GU;
  const int fb_gu = (a.I_max + kFeatPerWG / KSG * RG - 1) / (kFeatPerWG / KSG * RG);
  constexpr int KSD = MOE_STREAM_KSPLIT_DN;
  const int fb_dn = (a.H + kFeatPerWG / KSD * RD - 1) / (kFeatPerWG / KSD * RD);
  const bool f32 = a.wdt == MOE_F32;
  const bool yf32 = a.y_dt == MOE_F32;
  const dim3 blk(256);
  if (a.wdt == MOE_MXFP4) {
    constexpr int U = MOE_STREAM_MX_U, MG = MOE_STREAM_MX_ROWS_GU, MD = MOE_STREAM_MX_ROWS_DN;
    const int fg = (a.I_max + kFeatPerWG * MG - 1) / (kFeatPerWG * MG);
    const int fd = (a.H + kFeatPerWG * MD - 1) / (kFeatPerWG * MD);
    hipLaunchKernelGGL((k_gateup_stream_mx<MG, U>), dim3(stream_grid(a.max_tiles, fg)), blk, 0, s, a, fg);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (mid_event && (e = hipEventRecord(mid_event, s)) != hipSuccess) return e;
    if (yf32)
      hipLaunchKernelGGL((k_down_stream_mx<true, MD, U>), dim3(stream_grid(a.max_tiles, fd)), blk, 0, s, a, fd);
    else
      hipLaunchKernelGGL((k_down_stream_mx<false, MD, U>), dim3(stream_grid(a.max_tiles, fd)), blk, 0, s, a, fd);
    return hipGetLastError();
  }
  const int fb_gu1 = (a.I_max + kFeatPerWG / KSG - 1) / (kFeatPerWG / KSG);
  if (f32)
    hipLaunchKernelGGL((k_gateup_stream<true, 1>), dim3(stream_grid(a.max_tiles, fb_gu1)), blk, 0, s, a, fb_gu1);
  else
    hipLaunchKernelGGL((k_gateup_stream<false, RG>), dim3(stream_grid(a.max_tiles, fb_gu)), blk, 0, s, a, fb_gu);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (mid_event && (err = hipEventRecord(mid_event, s)) != hipSuccess) return err;
  const int fb_dn1 = (a.H + kFeatPerWG / KSD - 1) / (kFeatPerWG / KSD);
  if (f32 && yf32)
    hipLaunchKernelGGL((k_down_stream<true, true, 1>), dim3(stream_grid(a.max_tiles, fb_dn1)), blk, 0, s, a, fb_dn1);
  else if (f32)
    hipLaunchKernelGGL((k_down_stream<true, false, 1>), dim3(stream_grid(a.max_tiles, fb_dn1)), blk, 0, s, a, fb_dn1);
  else if (a.H % (16 * RDW) == 0) {
    // 16 RDW output features a wavefront (r1_decode: down 0.750 -> 0.728 ms against 16 RD):
    // each workgroup loads its tile's h rows once for twice the weight rows
    const int fb_dw = a.H / (kFeatPerWG / KSD * RDW);
    if (yf32)
      hipLaunchKernelGGL((k_down_stream<false, true, RDW>), dim3(stream_grid(a.max_tiles, fb_dw)), blk, 0, s, a, fb_dw);
    else
      hipLaunchKernelGGL((k_down_stream<false, false, RDW>), dim3(stream_grid(a.max_tiles, fb_dw)), blk, 0, s, a, fb_dw);
  } else if (yf32)
    hipLaunchKernelGGL((k_down_stream<false, true, RD>), dim3(stream_grid(a.max_tiles, fb_dn)), blk, 0, s, a, fb_dn);
  else
    hipLaunchKernelGGL((k_down_stream<false, false, RD>), dim3(stream_grid(a.max_tiles, fb_dn)), blk, 0, s, a, fb_dn);
  return hipGetLastError();
}

}  // namespace moe
