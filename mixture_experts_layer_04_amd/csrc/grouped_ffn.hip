// Grouped SwiGLU expert FFN: for every expert (group), h = SiLU(x Wg^T) * (x Wu^T) on its
// rows, then y = h W2^T -- the per-expert FFN of moe_ffn ("Decoding Trillion-Parameter
// MoE LLMs", section "Routing: Top-K Experts Plus a Shared Expert") run as one grouped
// GEMM pair with SwiGLU fused into the gate/up epilogue, as in the grouped GEMM of
// "GC-MoE: Overlapping Expert-Parallel Token Dispatch with FP8/FP4 Grouped GEMM via CUDA
// Green Contexts" (key_changes, fourth item). Decode is bound by streaming the weights of
// the touched experts ("why_it_matters" of the same record).
//
// Work is described by a device-side tile list (permute.hip): each tile is up to tile_m
// rows of one group. Launch grids use a host-side upper bound on the tile count; surplus
// workgroups exit at once, so no host synchronisation is needed.
//
// Kernel families, chosen per call: streaming kernels (ffn_stream.hip), the LDS-tiled bf16 /
// MXFP4 kernel (ffn_tiled.hip), the fp8 / INT8 kernel (ffn_fp8.hip), the W4A4 kernel
// (ffn_w4a4.hip), and plain dot products for bf16 / fp32 shapes that are multiples of 8 but
// not of 64 (ffn_generic.hip).
#include "ffn_common.h"

namespace moe {

bool ffn_shape_ok(moe_dtype wdt, int32_t H, int32_t I) {
  switch (wdt) {
    // multiples of 64 go to the MFMA kernels, other multiples of 8 to ffn_generic.hip
    case MOE_F32:
    case MOE_BF16: return H % 8 == 0 && I % 8 == 0;
    case MOE_FP8_E4M3:
    case MOE_INT8: return H % kF8Feat == 0 && I % kF8Feat == 0;
    // the tiled kernel's weight-row blocks, and dword-aligned scale bytes of every row
    case MOE_MXFP4: return H % kTiledN == 0 && I % 128 == 0;
    // 128-element K blocks of the FP4 instruction
    case MOE_MXFP4_A4: return H % 128 == 0 && I % 128 == 0;
  }
  return false;
}

int32_t ffn_tile_m(moe_dtype wdt, int32_t rows, int32_t groups, int32_t H, int32_t I_routed,
                   int32_t I_shared) {
  if (wdt == MOE_FP8_E4M3 || wdt == MOE_INT8) return kF8TileM;
  if (wdt == MOE_MXFP4_A4) return kTiledM;
  // MXFP4: streaming kernels for few rows per expert where the shapes allow, else tiled
  if (wdt == MOE_MXFP4)
    return (int64_t)rows <= 32 * (int64_t)groups && ffn_stream_mx_ok(H, I_routed) &&
                   (I_shared == 0 || ffn_stream_mx_ok(H, I_shared))
               ? kStreamTileM
               : kTiledM;
  // Few rows per expert: stream the weights (each weight element read once per tile of
  // <= 16 rows). Many rows: LDS-tiled GEMM with 256-row tiles (256 weight rows a
  // workgroup) where H and I allow, else 128-row tiles.
  auto tiled_ok = [&](int n) {
    return H % n == 0 && I_routed % (n / 2) == 0 && I_shared % (n / 2) == 0;
  };
  if (wdt == MOE_BF16 && (int64_t)rows > 32 * (int64_t)groups) {
    if (tiled_ok(kTiledNB)) return kTiledMB;
    if (tiled_ok(kTiledN)) return kTiledM;
  }
  return kStreamTileM;
}

int32_t ffn_stream_tile_rows() { return kStreamTileM; }

size_t ffn_scratch_bytes(moe_dtype wdt, int32_t rows_total, int32_t H, int32_t I_routed,
                         int32_t I_shared) {
  const int32_t I_max = I_shared > I_routed ? I_shared : I_routed;
  if (ffn_generic(wdt, H, I_routed, I_shared))  // h kept fp32
    return ((size_t)rows_total * I_max * 4 + 255) / 256 * 256;
  if (wdt == MOE_FP8_E4M3 || wdt == MOE_INT8) {
    const size_t q = ((size_t)rows_total * I_max + 255) / 256 * 256;
    return q + ((size_t)rows_total * (I_max / kF8K) * sizeof(float) + 255) / 256 * 256;
  }
  if (wdt == MOE_MXFP4_A4) {
    const size_t q = ((size_t)rows_total * (I_max / 2) + 255) / 256 * 256;
    return q + ((size_t)rows_total * (I_max / 32) + 255) / 256 * 256;
  }
  if (wdt == MOE_BF16) {  // h as bf16 plus its MXFP4-coded residual (ffn_common.h)
    const size_t hi = ((size_t)rows_total * I_max * 2 + 255) / 256 * 256;
    const size_t lo = ((size_t)rows_total * (I_max / 2) + 255) / 256 * 256;
    return hi + lo + ((size_t)rows_total * lo_sstride(I_max) + 255) / 256 * 256;
  }
  const size_t hb = (wdt == MOE_F32) ? 4 : 2;
  return ((size_t)rows_total * I_max * hb + 255) / 256 * 256;
}

hipError_t launch_grouped_ffn(FfnArgs a, void* scratch, hipStream_t s, hipEvent_t mid_event) {
  if (a.max_tiles <= 0) {
    return mid_event ? hipEventRecord(mid_event, s) : hipSuccess;
  }
  a.h = scratch;
  if (ffn_generic(a.wdt, a.H, a.bank[0].I, a.has_shared ? a.bank[1].I : 0))
    return launch_ffn_generic(a, s, mid_event);
  if (a.wdt == MOE_FP8_E4M3 || a.wdt == MOE_INT8) {
    a.h_scale = reinterpret_cast<float*>(reinterpret_cast<char*>(scratch) +
                                         ((size_t)a.rows_total * a.I_max + 255) / 256 * 256);
    return launch_ffn_fp8(a, s, mid_event);
  }
  if (a.wdt == MOE_MXFP4_A4) {
    a.h_xs = reinterpret_cast<uint8_t*>(scratch) + ((size_t)a.rows_total * (a.I_max / 2) + 255) / 256 * 256;
    return launch_ffn_w4a4(a, s, mid_event);
  }
  if (a.wdt == MOE_BF16) {
    char* p = reinterpret_cast<char*>(scratch) + ((size_t)a.rows_total * a.I_max * 2 + 255) / 256 * 256;
    a.h_lo = reinterpret_cast<uint8_t*>(p);
    a.h_lo_s = a.h_lo + ((size_t)a.rows_total * (a.I_max / 2) + 255) / 256 * 256;
  }
  if ((a.tile_m == kTiledM || a.tile_m == kTiledMB) && (a.wdt == MOE_BF16 || a.wdt == MOE_MXFP4))
    return launch_ffn_tiled(a, s, mid_event);
  return launch_ffn_stream(a, s, mid_event);
}

}  // namespace moe
