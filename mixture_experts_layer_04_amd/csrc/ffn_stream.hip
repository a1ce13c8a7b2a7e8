// Streaming grouped-FFN kernels (few rows per expert, e.g. decode), which are bound by
// streaming the weights of the touched experts ("GC-MoE: Overlapping Expert-Parallel
// Token Dispatch with FP8/FP4 Grouped GEMM via CUDA Green Contexts", why_it_matters).
// The weights are the MFMA A operand (16 output features per wavefront), the <= 16 rows
// of the tile the B operand. Each lane loads 32 contiguous bytes of its weight row per
// step (a full 128-B line per 4 lanes) straight from HBM into registers: a weight element
// is read exactly once per tile and never staged in LDS. bf16 uses
// v_mfma_f32_16x16x32_bf16, fp32 v_mfma_f32_16x16x4_f32. Because a dot product may be
// summed in any order, the K index carried by lane group kq and register slot j is
// k0 + 16*kq + j (bf16) -- the same map for A and B -- which makes every load contiguous.
// Two wavefronts of a workgroup share one group of weight rows, each streaming half of
// its K range; their fp32 partial sums meet in LDS and are added in K order (shorter
// streams per wavefront measured 1-2% faster than whole rows, longer ones slower).
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
#ifndef MOE_STREAM_UNROLL_GU
#define MOE_STREAM_UNROLL_GU 2
#endif
#ifndef MOE_STREAM_ROWS_GU  // 16-row weight groups per wavefront (bf16)
#define MOE_STREAM_ROWS_GU 4
#endif
#ifndef MOE_STREAM_ROWS_DN
#define MOE_STREAM_ROWS_DN 1
#endif
#ifndef MOE_STREAM_UNROLL_DN
#define MOE_STREAM_UNROLL_DN 8
#endif
#ifndef MOE_STREAM_DN_LDS  // bf16 down with the tile's h rows staged in LDS (where I allows)
#define MOE_STREAM_DN_LDS 1
#endif
#ifndef MOE_STREAM_KSPLIT_GU  // gate/up: wavefronts that share one row group, each a K range
#define MOE_STREAM_KSPLIT_GU 2
#endif
#ifndef MOE_STREAM_KSPLIT_DN  // the same for down
#define MOE_STREAM_KSPLIT_DN 2
#endif
// Weight fragment: ordinary cached loads (on MI355X they measured faster than
// non-temporal ones for this many-rows-at-once pattern).
__device__ __forceinline__ Frag32 load_w(const void* p) { return load_c(p); }
// Activation fragment of a row; lanes of padding rows (beyond the tile's rows) load
// nothing and contribute zeros to columns that are never stored.
__device__ __forceinline__ Frag32 load_x(const void* p, bool valid) {
  if (valid) return load_c(p);
  Frag32 z;
  z.lo = u32x4{0, 0, 0, 0};
  z.hi = u32x4{0, 0, 0, 0};
  return z;
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
  const int tile_id = blockIdx.x / fb_per_tile;
  const int fb = blockIdx.x - tile_id * fb_per_tile;
  if (tile_id >= *a.ntiles) return;
  const Tile tl = a.tiles[tile_id];
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
  const int64_t lane_off = (int64_t)kq * kLane * esz;
  const char* wg[R];
  const char* wu[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    wg[r] = w13 + (int64_t)(f0 + 16 * r + m) * H * esz + lane_off;
    wu[r] = w13 + (int64_t)(I + f0 + 16 * r + m) * H * esz + lane_off;
  }
  const char* xr = reinterpret_cast<const char*>(a.a) + src * H * esz + lane_off;
  f32x4 accg[R], accu[R];
#pragma unroll
  for (int r = 0; r < R; ++r) accg[r] = accu[r] = f32x4{0, 0, 0, 0};
  const int nst = H / kStep;
  const int kbeg = active ? (ks * nst / KS) * kStep : 0;
  const int kend = active ? ((ks + 1) * nst / KS) * kStep : 0;
  const int kmain = kend - (kend - kbeg) % (kStep * U);
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
  if (xv) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      f32x4 hv;
#pragma unroll
      for (int i = 0; i < 4; ++i) hv[i] = silu_mul(accg[r][i], accu[r][i]);
      store4<kF32>(a.h, (int64_t)(tl.row0 + m) * a.I_max + f0 + 16 * r + kq * 4, hv);
    }
  }
}

// Down projection. Workgroup = (tile, block of 64 R / KS output features of H); wavefronts
// w = KS q + ks compute R groups of 16 output features over K range ks, reusing one h
// fragment per K step.
template <bool kF32, bool kYF32, int R>
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
  constexpr int KS = MOE_STREAM_KSPLIT_DN;
  static_assert(4 % KS == 0, "K split divides the workgroup");
  const int ks = wave % KS;
  const int f0 = (fb * (4 / KS) + wave / KS) * 16 * R;
  if (KS == 1 && f0 >= H) return;
  const bool active = f0 < H;
  const int m = l & 15, kq = l >> 4;
  const int esz = kF32 ? 4 : 2;
  constexpr int kStep = kF32 ? 32 : 64;
  constexpr int kLane = kStep / 4;
  constexpr int U = MOE_STREAM_UNROLL_DN;
  const int64_t lane_off = (int64_t)kq * kLane * esz;
  // this wavefront's K range [kbeg, kend), whole K steps
  const int nst = I / kStep;
  const int kbeg = active ? (ks * nst / KS) * kStep : 0;
  const int kend = active ? ((ks + 1) * nst / KS) * kStep : 0;
  const bool xv = m < tl.nrows;
  const char* w2 = reinterpret_cast<const char*>(a.bank[bank].w2) + ge * (int64_t)H * I * esz;
  const char* wr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) wr[r] = w2 + (int64_t)(f0 + 16 * r + m) * I * esz + lane_off;
  const char* hr = reinterpret_cast<const char*>(a.h) +
                   (int64_t)(tl.row0 + (xv ? m : 0)) * a.I_max * esz + lane_off;
  f32x4 acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = f32x4{0, 0, 0, 0};
  const int kmain = kend - (kend - kbeg) % (kStep * U);
  for (int k0 = kbeg; k0 < kmain; k0 += kStep * U) {
    Frag32 fw[U][R], fh[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t o = (int64_t)(k0 + u * kStep) * esz;
#pragma unroll
      for (int r = 0; r < R; ++r) fw[u][r] = load_w(wr[r] + o);
      fh[u] = load_x(hr + o, xv);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = mma<kF32>(fw[u][r], fh[u], acc[r]);
  }
  for (int k0 = kmain; k0 < kend; k0 += kStep) {
    const int64_t o = (int64_t)k0 * esz;
    const Frag32 fh = load_x(hr + o, xv);
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = mma<kF32>(load_w(wr[r] + o), fh, acc[r]);
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

// Down projection, bf16, with the tile's h rows staged in LDS: the workgroup's four
// wavefronts (four groups of 16 output features) share each 512-element K chunk of the
// 16 h rows, which goes global -> LDS by DMA (each wavefront one 1-KB row piece of four
// rows) through two buffers, instead of every wavefront loading it into registers. Lane l
// of the DMA of row p takes the 16-B piece l ^ p of the row, so that the 16 rows' reads of
// one lane group fall in different banks. Needs I % 512 == 0.
constexpr int kDnLdsK = 512;  // K elements per chunk (8 MFMA steps)
template <bool kYF32>
__global__ void __launch_bounds__(256) k_down_stream_lds(FfnArgs a, int fb_per_tile) {
  constexpr int U = kDnLdsK / 64;
  constexpr int CB = 16 * kDnLdsK * 2;  // bytes of a chunk
  __shared__ __attribute__((aligned(1024))) char hs[2 * CB];
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int tile_id = blockIdx.x / fb_per_tile;
  const int fb = blockIdx.x - tile_id * fb_per_tile;
  if (tile_id >= *a.ntiles) return;
  const Tile tl = a.tiles[tile_id];
  const int bank = tl.group < a.E ? 0 : 1;
  const int64_t ge = tl.group < a.E ? tl.group : 0;
  const int I = a.bank[bank].I;
  const int H = a.H;
  const int f0 = (fb * 4 + wave) * 16;
  const bool active = f0 < H;
  const int m = l & 15, kq = l >> 4;
  const bool xv = m < tl.nrows;
  const char* wr = reinterpret_cast<const char*>(a.bank[bank].w2) + ge * (int64_t)H * I * 2 +
                   (int64_t)(active ? f0 + m : 0) * I * 2 + kq * 32;
  const char* hsrc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p = 4 * wave + j;
    const int rr = p < tl.nrows ? p : (tl.nrows > 0 ? tl.nrows - 1 : 0);  // padding rows: any valid row
    hsrc[j] = reinterpret_cast<const char*>(a.h) + (int64_t)(tl.row0 + rr) * a.I_max * 2 + (l ^ p) * 16;
  }
  auto issue = [&](int c) {
    char* dst = hs + (c & 1) * CB;
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16(hsrc[j] + (int64_t)c * kDnLdsK * 2, dst + (4 * wave + j) * 1024);
  };
  const int nch = I / kDnLdsK;
  f32x4 acc = f32x4{0, 0, 0, 0};
  issue(0);
  for (int c = 0; c < nch; ++c) {
    Frag32 fw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) fw[u] = load_w(wr + (int64_t)(c * kDnLdsK + u * 64) * 2);
    wait_vmcnt<2 * U>();  // this wavefront's DMA of chunk c (issued before the 2 U weight loads)
    __builtin_amdgcn_s_barrier();  // ... and every other wavefront's; chunk c - 1 is read
    if (c + 1 < nch) issue(c + 1);
    const char* hb = hs + (c & 1) * CB + m * 1024;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      Frag32 fh;
      fh.lo = *reinterpret_cast<const u32x4*>(hb + (((u * 8 + kq * 2) ^ m) << 4));
      fh.hi = *reinterpret_cast<const u32x4*>(hb + (((u * 8 + kq * 2 + 1) ^ m) << 4));
      acc = mma_bf16(fw[u], fh, acc);
    }
  }
  if (xv && active) store4<kYF32>(a.y, (int64_t)(tl.row0 + m) * H + f0 + kq * 4, acc);
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
  const int tile_id = blockIdx.x / fb_per_tile;
  const int fb = blockIdx.x - tile_id * fb_per_tile;
  if (tile_id >= *a.ntiles) return;
  const Tile tl = a.tiles[tile_id];
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
  const int row = tl.row0 + (xv ? m : 0);
  const int64_t src = a.a_rowmap ? a.a_rowmap[row] : row;
  const char* xr = reinterpret_cast<const char*>(a.a) + src * H * 2 + 64 * kq;
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
  for (int k0 = 0, c = 0; k0 < H; k0 += 256 * U, ++c) {
    MxCodes<U> wg[R], wu[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      wg[r] = load_mx<U>(cg[r] + k0 / 2, sg[r] + k0 / 32);
      wu[r] = load_mx<U>(cu[r] + k0 / 2, su[r] + k0 / 32);
    }
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
        accg[r] = mma_mx_part<U>(wg[r], x4, i, kq, accg[r]);
        accu[r] = mma_mx_part<U>(wu[r], x4, i, kq, accu[r]);
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
  const int tile_id = blockIdx.x / fb_per_tile;
  const int fb = blockIdx.x - tile_id * fb_per_tile;
  if (tile_id >= *a.ntiles) return;
  const Tile tl = a.tiles[tile_id];
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
  const char* hr = reinterpret_cast<const char*>(a.h) +
                   (int64_t)(tl.row0 + (xv ? m : 0)) * a.I_max * 2 + 64 * kq;
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
  for (int k0 = 0, c = 0; k0 < I; k0 += 256 * U, ++c) {
    MxCodes<U> w[R];
#pragma unroll
    for (int r = 0; r < R; ++r) w[r] = load_mx<U>(cw[r] + k0 / 2, sw[r] + k0 / 32);
#if MOE_STREAM_MX_LDS
    wait_vmcnt<R * (2 * U + 1)>();
    __builtin_amdgcn_s_barrier();
    if (k0 + 256 * U < I) issue(c + 1);
#pragma unroll
    for (int i = 0; i < 2 * U; ++i) {
      u32x4 x4[4];
      read_x_mx_lds(xs + (c & 1) * kMxChunk, m, kq, i, x4);
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = mma_mx_part<U>(w[r], x4, i, kq, acc[r]);
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
  constexpr int RG = MOE_STREAM_ROWS_GU, RD = MOE_STREAM_ROWS_DN;
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
    hipLaunchKernelGGL((k_gateup_stream_mx<MG, U>), dim3(a.max_tiles * fg), blk, 0, s, a, fg);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (mid_event && (e = hipEventRecord(mid_event, s)) != hipSuccess) return e;
    if (yf32)
      hipLaunchKernelGGL((k_down_stream_mx<true, MD, U>), dim3(a.max_tiles * fd), blk, 0, s, a, fd);
    else
      hipLaunchKernelGGL((k_down_stream_mx<false, MD, U>), dim3(a.max_tiles * fd), blk, 0, s, a, fd);
    return hipGetLastError();
  }
  if (f32)
    hipLaunchKernelGGL((k_gateup_stream<true, 1>), dim3(a.max_tiles * ((a.I_max + kFeatPerWG / KSG - 1) / (kFeatPerWG / KSG))), blk, 0, s, a, (a.I_max + kFeatPerWG / KSG - 1) / (kFeatPerWG / KSG));
  else
    hipLaunchKernelGGL((k_gateup_stream<false, RG>), dim3(a.max_tiles * fb_gu), blk, 0, s, a, fb_gu);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (mid_event && (err = hipEventRecord(mid_event, s)) != hipSuccess) return err;
  const int fb_dn1 = (a.H + kFeatPerWG / KSD - 1) / (kFeatPerWG / KSD);
  if (f32 && yf32)
    hipLaunchKernelGGL((k_down_stream<true, true, 1>), dim3(a.max_tiles * fb_dn1), blk, 0, s, a, fb_dn1);
  else if (f32)
    hipLaunchKernelGGL((k_down_stream<true, false, 1>), dim3(a.max_tiles * fb_dn1), blk, 0, s, a, fb_dn1);
  else if (MOE_STREAM_DN_LDS && a.bank[0].I % kDnLdsK == 0 && a.bank[1].I % kDnLdsK == 0) {
    const int fbl = (a.H + kFeatPerWG - 1) / kFeatPerWG;
    if (yf32)
      hipLaunchKernelGGL((k_down_stream_lds<true>), dim3(a.max_tiles * fbl), blk, 0, s, a, fbl);
    else
      hipLaunchKernelGGL((k_down_stream_lds<false>), dim3(a.max_tiles * fbl), blk, 0, s, a, fbl);
  } else if (yf32)
    hipLaunchKernelGGL((k_down_stream<false, true, RD>), dim3(a.max_tiles * fb_dn), blk, 0, s, a, fb_dn);
  else
    hipLaunchKernelGGL((k_down_stream<false, false, RD>), dim3(a.max_tiles * fb_dn), blk, 0, s, a, fb_dn);
  return hipGetLastError();
}

}  // namespace moe
