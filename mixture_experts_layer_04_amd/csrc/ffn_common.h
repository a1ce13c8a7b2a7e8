// Device helpers and constants shared by the grouped-FFN kernel files (ffn_stream.hip,
// ffn_tiled.hip, ffn_fp8.hip), and the launcher each of them gives grouped_ffn.hip.
// Internal; not part of the ABI.
#pragma once

#include "moe_internal.h"

namespace moe {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Rows per tile of each kernel family; the tile list of a call is built for one of them.
constexpr int kStreamTileM = 16;   // streaming kernels (few rows per expert)
constexpr int kTiledM = 128;       // LDS-tiled bf16 / MXFP4 kernel
constexpr int kTiledN = 128;       // its weight rows per workgroup (gate/up: 64 features)
constexpr int kTiledMB = 256;      // LDS-tiled bf16 kernel with 256 x 256 tiles
constexpr int kTiledNB = 256;      // (where H % 256 == 0 and I % 128 == 0)
constexpr int kF8TileM = 128;      // fp8 kernel
constexpr int kF8Feat = 128;       // fp8 output features per workgroup = one scale block
constexpr int kF8K = 128;          // fp8 K block = one scale block

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// LDS byte offset of logical 16-B chunk c of tile row r (each 16-row group takes
// eight 256-B lines, row j and row 8 + j share line j, chunks XOR-swizzled by row & 7;
// ffn_tiled.hip describes it).
__device__ __forceinline__ int lds_off(int r, int c) {
  return (r >> 4) * 2048 + (r & 7) * 256 + ((r >> 3) & 1) * 128 + ((c ^ (r & 7)) << 4);
}
// Row and logical chunk that lane l of 1-KB DMA block q writes.
__device__ __forceinline__ void dma_slot(int q, int l, int* r, int* c) {
  const int half = (l >> 3) & 1;
  *r = (q >> 1) * 16 + (q & 1) * 4 + (l >> 4) + 8 * half;
  *c = (l & 7) ^ (*r & 7);
}

typedef __attribute__((address_space(3))) void lds_void;

// 16 B per lane from global memory into LDS at lds + 16 * lane (a device-only wrapper: the
// target builtin must not appear in code the host pass instantiates).
__device__ __forceinline__ void dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, 0);
}
// The same with the non-temporal hint (nt): for data read once (weights streamed past
// every other user), which streams from HBM faster than a cached request when a
// wavefront's lanes cover whole 128-B lines.
__device__ __forceinline__ void dma16nt(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, 2);
}
// 4 B per lane from global memory into LDS at lds + 4 * lane (device-only wrapper).
__device__ __forceinline__ void dma4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 4, 0, 0);
}
// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// E8M0 scale byte -> its power of two as fp32 (0xFF is NaN; 0 is 2^-127, a subnormal).
// Written as selects: with early returns the compiler branched on them lane by lane.
__device__ __forceinline__ float e8m0_f32(uint32_t c) {
  uint32_t bits = c << 23;
  bits = c == 0u ? 0x00400000u : bits;     // 2^-127
  bits = c == 0xFFu ? 0x7FC00000u : bits;  // NaN
  return __uint_as_float(bits);
}
// The same in two instructions for codes 0..254 (exact, 0 giving 2^-127); code 0xFF gives
// +Inf instead of NaN, so that a block with a NaN scale decodes to infinities (non-zero
// codes) and NaNs (zero codes). For the tiled MXFP4 kernel's weight scales (ep32_mxfp4
// gate/up 0.913 -> 0.890 ms against e8m0_f32) and h's residual, whose writer emits 0..254.
__device__ __forceinline__ float e8m0_f32_fast(uint32_t c) {
  return __uint_as_float(max(c << 23, 0x00400000u));
}

// Eight E2M1 values (one 32-bit word, low nibble first) times their E8M0 block scale, as
// the bf16 fragment of one MFMA k-step (v_cvt_scalef32_pk_bf16_fp4 is exact: every
// E2M1 value times a power of two in range is a bf16).
__device__ __forceinline__ bf16x8 e2m1x8_bf16(uint32_t w, float scale) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// E2M1 code of v (already divided by the block scale): nearest of 0, .5, 1, 1.5, 2, 3, 4,
// 6, ties to the even code, larger magnitudes to 6; the sign in bit 3 (also for zero).
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fabsf(v);
  const uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
                     (a >= 3.5f) + (a > 5.0f);
  return c | ((__float_as_uint(v) >> 28) & 0x8u);
}

// OCP MX shared-scale exponent e of a block from its amax (a non-negative fp32):
// floor(log2 amax) - 2, 2 being the exponent of E2M1's largest value; 0 for a zero block,
// clamped below at -127.
__device__ __forceinline__ int mx_exponent(float amax) {
  const int be = (int)(__float_as_uint(amax) >> 23);  // biased exponent (amax >= 0)
  if (amax == 0.0f) return 0;
  if (be == 0) return -127;                            // subnormal amax: below 2^-125
  const int e = be - 127 - 2;
  return e < -127 ? -127 : e;
}

__device__ __forceinline__ float exp2i(int e) {  // 2^e for e in [-127, 127], exact
  return e >= -126 ? __uint_as_float((uint32_t)(e + 127) << 23) : __uint_as_float(0x00400000u);
}

// ------------------------------------------------ SwiGLU output of bf16 expert banks
// With bf16 weights, h = SiLU(g) * u goes to the down GEMM as two parts: hi = bf16(h), and
// the residual lo = h - hi (exact in fp32) coded as MXFP4 -- E2M1 codes, two a byte
// (element 2i in the low nibble of byte i), and an E8M0 scale per 32 features. The down
// GEMM multiplies both parts with the same weight fragments. A bf16 h alone is off by up
// to 2^-9 of each element; with the residual, by at most a quarter of the residual's block
// scale unit, which keeps heavy-tailed outputs within the bf16 tolerance (a bf16 h alone
// does not: it adds about a third to the error the bf16 output storage already makes).
// Scratch layout, per grouped row: hi [I_max] bf16 (the h buffer), lo codes [I_max / 2]
// bytes, lo scales [lo_sstride(I_max)] bytes (padded so rows start 16-B aligned and every
// aligned dword of scales lies inside the row).
__host__ __device__ inline int32_t lo_sstride(int32_t I_max) { return (I_max / 32 + 15) / 16 * 16; }

// bf16 value and MXFP4 residual of h: returns hi's bits, sets *lo = h - hi (exact).
__device__ __forceinline__ uint16_t split_bf16(float h, float* lo) {
  const uint16_t b = f32_to_bf16(h);
  *lo = h - bf16_to_f32(b);
  return b;
}

// The work item (tile, feature block) of this workgroup when a launch's items are dealt to
// the 8 XCDs in contiguous chunks (workgroup b runs on XCD b mod 8): chunk x goes to XCD
// x, and inside a chunk the tiles of one tile block run side by side per feature block,
// so that the items sharing a tile's rows (or a group's weights) meet in one L2. The grid
// must be a whole number of rounds of 8 covering ntiles * fb_per_tile items (xcd_grid).
// Returns false for a workgroup without an item.
constexpr int kXcdCount = 8;  // MI355X
__device__ __forceinline__ bool xcd_chunked_item(const FfnArgs& a, int fb_per_tile, int* fb,
                                                 Tile* tl) {
  const int nitems = *a.ntiles * fb_per_tile;
  const int chunk = (nitems + kXcdCount - 1) / kXcdCount;
  const int slot = blockIdx.x / kXcdCount;
  const int item = (blockIdx.x % kXcdCount) * chunk + slot;
  if (slot >= chunk || item >= nitems) return false;
  const Tile tb = a.tiles[item / fb_per_tile];
  const int o = item - tb.blk0 * fb_per_tile;
  *fb = o / tb.nblk;
  *tl = a.tiles[tb.blk0 + (o - *fb * tb.nblk)];
  return true;
}
// Workgroups for max_tiles * fb_per_tile items, in whole rounds of the XCD count.
inline int xcd_grid(int max_tiles, int fb_per_tile) {
  return (max_tiles * fb_per_tile + kXcdCount - 1) / kXcdCount * kXcdCount;
}

// A compile-time int as a value, so that a generic lambda can be instantiated per count.
template <int N>
struct IntC {
  static constexpr int value = N;
};

// Launchers of the kernel families (FfnArgs as set up by launch_grouped_ffn; mid_event,
// if not null, is recorded between the gate/up and the down launches).
hipError_t launch_ffn_stream(const FfnArgs& a, hipStream_t s, hipEvent_t mid_event);
// Whether the MXFP4 streaming kernels take this H and I (multiples of their K iteration).
bool ffn_stream_mx_ok(int32_t H, int32_t I);
hipError_t launch_ffn_tiled(const FfnArgs& a, hipStream_t s, hipEvent_t mid_event);
hipError_t launch_ffn_fp8(const FfnArgs& a, hipStream_t s, hipEvent_t mid_event);
hipError_t launch_ffn_w4a4(const FfnArgs& a, hipStream_t s, hipEvent_t mid_event);
hipError_t launch_ffn_generic(const FfnArgs& a, hipStream_t s, hipEvent_t mid_event);

}  // namespace moe
