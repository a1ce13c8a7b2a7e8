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

}  // namespace moe
