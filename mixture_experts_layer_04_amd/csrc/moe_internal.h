// Internal declarations of the MoE layer library: device helpers, the tile list
// shared by the permute and grouped-GEMM kernels, and the launchers each .hip file
// provides to the C-ABI layer (moe_api.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// ------------------------------------------------------------------------ vector types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// bf16 bit pattern <-> fp32 (bf16 is the upper half of an fp32).
__device__ __forceinline__ float bf16_lo(uint32_t two) { return __uint_as_float(two << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t two) { return __uint_as_float(two & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
// fp32 -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ------------------------------------------------------------------------- tile list
// A row range of one group (expert): rows [row0, row0 + nrows) of the permuted row
// space, all belonging to `group`. Groups 0..E-1 are routed experts; group E, when
// present, is the shared expert. Built on the device by the permute scan kernel.
// Consecutive tiles of one group are also cut into blocks of up to kTileBlock tiles; the
// tiled GEMMs order their work items block by block (see ffn_tiled.hip).
#ifndef MOE_TILE_BLOCK
#define MOE_TILE_BLOCK 8
#endif
constexpr int kTileBlock = MOE_TILE_BLOCK;
struct Tile {
  int32_t group;
  int32_t row0;
  int32_t nrows;
  int32_t blk0;    // index of the first tile of this tile's block
  int32_t nblk;    // tiles in that block (1 .. kTileBlock)
  int32_t pad[3];  // 32-byte entries
};

// Upper bound of the tile count for n_rows rows in n_groups groups with tiles of m rows.
inline int64_t max_tiles(int64_t n_rows, int64_t n_groups, int64_t m) {
  return n_rows / m + n_groups;
}

// ---------------------------------------------------------------------- expert banks
// Device-side view of one bank of experts (routed: E experts; shared: 1).
struct BankView {
  const void* w13;
  const void* w13_scale;
  const void* w2;
  const void* w2_scale;
  int32_t I;
};

// Everything the grouped FFN kernels need for one call.
struct FfnArgs {
  moe_dtype wdt;          // weight format (both banks)
  moe_dtype act_dt;       // F32 or BF16 activation rows
  moe_dtype y_dt;         // F32 or BF16 output rows
  int32_t E;              // routed groups; group E is the shared bank when has_shared
  int32_t has_shared;
  int32_t H;
  int32_t I_max;          // row stride of h
  BankView bank[2];
  // activations: row r of the grouped row space reads a + map(r) * H, where
  // map(r) = a_rowmap ? a_rowmap[r] : r
  const void* a;
  const int32_t* a_rowmap;
  // fp8 / INT8 paths: activations pre-quantised to E4M3 or INT8 (a_q, [*, H]) with fp32
  // scales [*, H/128]
  const uint8_t* a_q;
  const float* a_qscale;
  // W4A4 path: activations as E2M1 codes (a_q, [*, H/2]) with E8M0 scales [*, H/32]
  const uint8_t* a_xs;
  void* h;                // [rows_total, I_max] intermediate (bf16, f32, or fp8/int8 + scales)
  float* h_scale;         // fp8 / INT8 paths: [rows_total, I_max/128]
  uint8_t* h_xs;          // W4A4 path: E8M0 scales of h [rows_total, I_max/32] (codes in h)
  uint8_t* h_lo;          // bf16 banks: MXFP4 codes of h's residual [rows_total, I_max/2]
  uint8_t* h_lo_s;        //   and their E8M0 scales [rows_total, lo_sstride(I_max)]
  void* y;                // [rows_total, H]
  const Tile* tiles;      // tile list (row chunks of `tile_m` rows)
  const int32_t* ntiles;  // device count of valid tiles
  int32_t max_tiles;      // launch bound on tiles
  int32_t tile_m;
  int32_t rows_total;
};

// ------------------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error. All enqueue on `s`.

// route.hip
size_t route_ws_bytes(int32_t T, int32_t H, int32_t E);
hipError_t launch_route(const void* x, moe_dtype x_dt, const void* wr, const float* bias,
                        int32_t T, int32_t H, int32_t E, int32_t k, moe_score_fn fn,
                        float scale, int32_t* topk_idx, float* topk_w, float* logits,
                        void* ws, hipStream_t s);

// permute.hip
size_t permute_ws_bytes(int32_t T, int32_t E);
// Counts, offsets, perm_src, inv_perm (and row_token[r] = token of row r, if non-NULL).
// If tiles != NULL also writes the tile list for tile_m-row chunks, including a shared
// group E of T rows starting at row T*k when with_shared.
hipError_t launch_permute_maps(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                               int32_t* counts, int32_t* offsets, int32_t* perm_src,
                               int32_t* inv_perm, int32_t* row_token, Tile* tiles,
                               int32_t* ntiles, int32_t tile_m, int32_t with_shared, void* ws,
                               hipStream_t s);
hipError_t launch_gather_rows(const void* x, int32_t elem_bytes, int32_t H,
                              const int32_t* perm_src, int32_t k, int32_t rows, void* x_perm,
                              hipStream_t s);
// Row map and tile list of the shared group alone (rows T*k .. T*k + T - 1, group E).
hipError_t launch_shared_group(int32_t T, int32_t k, int32_t E, int32_t tile_m, int32_t* row_token,
                               Tile* tiles, int32_t* ntiles, hipStream_t s);
// Hot and cold tile lists from the offsets (and the shared group E of T rows at row T*k):
// groups of more than cold_max rows in tm_hot-row tiles, the rest in tm_cold-row tiles.
hipError_t launch_split_tiles(const int32_t* offsets, int32_t E, int32_t T, int32_t k,
                              int32_t with_shared, int32_t cold_max, int32_t tm_hot, Tile* hot,
                              int32_t* n_hot, int32_t tm_cold, Tile* cold, int32_t* n_cold,
                              hipStream_t s);
// Tile list straight from a device offsets array (grouped FFN called on its own).
hipError_t launch_tiles_from_offsets(const int32_t* offsets, int32_t E, Tile* tiles,
                                     int32_t* ntiles, int32_t tile_m, hipStream_t s);

// grouped_ffn.hip
// Whether the grouped FFN kernels support this format and shape.
bool ffn_shape_ok(moe_dtype wdt, int32_t H, int32_t I);
// Rows per tile for a call: streaming (16) or tiled; I_shared = 0 when there is none.
int32_t ffn_tile_m(moe_dtype wdt, int32_t rows, int32_t groups, int32_t H, int32_t I_routed,
                   int32_t I_shared);
size_t ffn_scratch_bytes(moe_dtype wdt, int32_t rows_total, int32_t H, int32_t I_routed,
                         int32_t I_shared);
// Whether a bf16 / fp32 layer takes the plain dot-product kernels (H or an I not a
// multiple of 64; I_shared 0 without a shared expert).
bool ffn_generic(moe_dtype wdt, int32_t H, int32_t I_routed, int32_t I_shared);
// Rows per tile of the streaming kernels (the tile_m that selects them).
int32_t ffn_stream_tile_rows();
// Runs gate/up + SwiGLU and down for all tiles. `scratch` holds h (and fp8 staging).
// If mid_event is non-NULL it is recorded between the gate/up and the down launches.
hipError_t launch_grouped_ffn(FfnArgs a, void* scratch, hipStream_t s,
                              hipEvent_t mid_event = nullptr);
// fp8 path: per 1 x 128 block E4M3 quantisation of rows of a [n, H] bf16 matrix.
hipError_t launch_quant_rows_fp8(const void* x, int32_t n, int32_t H, uint8_t* q, float* qs,
                                 hipStream_t s);
// W8A8 path: per 1 x 128 block INT8 quantisation of rows of a [n, H] bf16 matrix.
hipError_t launch_quant_rows_int8(const void* x, int32_t n, int32_t H, int8_t* q, float* qs,
                                  hipStream_t s);
// W4A4 path: per 1 x 32 block MXFP4 quantisation of rows of a [n, H] bf16 matrix.
hipError_t launch_quant_rows_mxfp4(const void* x, int32_t n, int32_t H, uint8_t* q, uint8_t* qs,
                                   hipStream_t s);

// balance.hip
// In-place selection-bias update from per-expert routed counts (1 <= E <= 1024).
hipError_t launch_bias_update(const int32_t* counts, int32_t E, float u, float* bias,
                              hipStream_t s);

// combine.hip
hipError_t launch_combine(const void* y, moe_dtype y_dt, const int32_t* inv_perm,
                          const float* topk_w, int32_t T, int32_t k, int32_t H,
                          const void* shared, void* out, moe_dtype out_dt, hipStream_t s);

// probe.hip (measurement probes, not part of the layer)
hipError_t launch_probe_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_probe_mfma(moe_dtype dt, int64_t iters, uint32_t* sink, double* flops,
                             hipStream_t s);

}  // namespace moe
