// C ABI of the MoE layer library (include/moe.h): host-side argument validation,
// workspace sizing and carving, and the launch sequence of each entry point. Nothing here
// synchronises, copies to the host or allocates; every call only enqueues on `stream`.
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "moe_internal.h"

using namespace moe;

namespace {

thread_local char g_last_hip[256] = "";

moe_status hip_fail(hipError_t e, const char* where) {
  snprintf(g_last_hip, sizeof g_last_hip, "%s: %s (%d)", where, hipGetErrorString(e), (int)e);
  return MOE_ERR_HIP;
}

inline size_t up256(size_t v) { return (v + 255) / 256 * 256; }
inline bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool al256(const void* p) { return ((uintptr_t)p & 255u) == 0; }

size_t dt_bytes(moe_dtype d) { return d == MOE_F32 ? 4 : 2; }

// Sizes and formats a bank must satisfy.
moe_status check_bank(const moe_experts* w, int32_t H, bool need_scales) {
  if (!w->w13 || !w->w2) return MOE_ERR_NULL;
  if (w->E < 1 || w->H != H || w->I < 1) return MOE_ERR_SHAPE;
  switch (w->dtype) {
    case MOE_F32:
    case MOE_BF16:
      break;
    case MOE_FP8_E4M3:
    case MOE_INT8:
    case MOE_MXFP4:
    case MOE_MXFP4_A4:
      if (need_scales && (!w->w13_scale || !w->w2_scale)) return MOE_ERR_NULL;
      break;
    default:
      return MOE_ERR_DTYPE;
  }
  if (!ffn_shape_ok(w->dtype, H, w->I)) return MOE_ERR_SHAPE;
  if (!al16(w->w13) || !al16(w->w2)) return MOE_ERR_ALIGN;
  if ((w->w13_scale && !al16(w->w13_scale)) || (w->w2_scale && !al16(w->w2_scale)))
    return MOE_ERR_ALIGN;
  return MOE_OK;
}

// Activation dtype that goes with a weight dtype.
bool act_ok(moe_dtype act, moe_dtype wdt) {
  if (wdt == MOE_F32) return act == MOE_F32;
  if (wdt == MOE_BF16 || wdt == MOE_FP8_E4M3 || wdt == MOE_MXFP4 || wdt == MOE_MXFP4_A4 ||
      wdt == MOE_INT8)
    return act == MOE_BF16;
  return false;
}
bool io_dt_ok(moe_dtype d) { return d == MOE_F32 || d == MOE_BF16; }

// ------------------------------------------------------------------ layer plan

struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    size_t o = off;
    off += up256(bytes);
    return o;
  }
};

struct FfnPlan {
  int32_t tile_m = 0, max_tiles = 0, rows_total = 0, I_max = 0;
  size_t o_tiles = 0, o_ntiles = 0, o_scratch = 0, o_y = 0;
  moe_dtype y_dt = MOE_BF16;
};

void plan_ffn(Carve& c, FfnPlan& p, moe_dtype wdt, moe_dtype act, int32_t H, int32_t I_routed,
              int32_t I_shared, int32_t rows_routed, int32_t E, int32_t shared_rows, bool need_y) {
  const int32_t I_max = I_shared > I_routed ? I_shared : I_routed;
  p.rows_total = rows_routed + shared_rows;
  p.I_max = I_max;
  p.tile_m = ffn_tile_m(wdt, rows_routed, E, H, I_routed, I_shared);
  int64_t mt = max_tiles(rows_routed, E, p.tile_m);
  if (shared_rows) mt += (shared_rows + p.tile_m - 1) / p.tile_m;
  p.max_tiles = (int32_t)mt;
  // bf16 and fp32 banks: expert outputs stay fp32 until the combine rounds once (with
  // bf16 rows here the heavy-tailed SwiGLU outputs of small layers measured up to 2.5e-2 of
  // the output RMS, over the bf16 tolerance). fp8, INT8, MXFP4 and W4A4 banks, whose layer
  // outputs are held to 6e-2 (their codes differ by a step where the GPU's fp32 h and the
  // float64 one fall on either side of a rounding boundary), store them as bf16: one more
  // rounding of at most 2^-9 of each term, and half the bytes between the down projection
  // and the combine.
  (void)act;
  p.y_dt = (wdt == MOE_BF16 || wdt == MOE_F32) ? MOE_F32 : MOE_BF16;
  p.o_tiles = c.take((size_t)mt * sizeof(Tile));
  p.o_ntiles = c.take(sizeof(int32_t));
  p.o_scratch = c.take(ffn_scratch_bytes(wdt, p.rows_total, H, I_routed, I_shared));
  if (need_y) p.o_y = c.take((size_t)p.rows_total * H * dt_bytes(p.y_dt));
}

// Staging of quantised activations: fp8 or INT8 (codes [rows, H], fp32 scales
// [rows, H/128]) or W4A4 (E2M1 codes [rows, H/2], E8M0 scales [rows, H/32]).
struct QPlan {
  size_t o_q = 0, o_qs = 0;
};
void plan_quant(Carve& c, QPlan& q, moe_dtype wdt, int32_t rows, int32_t H) {
  if (wdt == MOE_FP8_E4M3 || wdt == MOE_INT8) {
    q.o_q = c.take((size_t)rows * H);
    q.o_qs = c.take((size_t)rows * (H / 128) * sizeof(float));
  } else if (wdt == MOE_MXFP4_A4) {
    q.o_q = c.take((size_t)rows * (H / 2));
    q.o_qs = c.take((size_t)rows * (H / 32));
  }
}
// Quantises the rows of x for the expert GEMMs (if the format needs it) and points f at them.
hipError_t quantise_acts(moe_dtype wdt, const void* x, int32_t rows, int32_t H, char* base,
                         const QPlan& q, FfnArgs& f, hipStream_t s) {
  if (wdt == MOE_FP8_E4M3 || wdt == MOE_INT8) {
    f.a_q = reinterpret_cast<const uint8_t*>(base + q.o_q);
    f.a_qscale = reinterpret_cast<const float*>(base + q.o_qs);
    if (wdt == MOE_INT8)
      return launch_quant_rows_int8(x, rows, H, reinterpret_cast<int8_t*>(base + q.o_q),
                                    reinterpret_cast<float*>(base + q.o_qs), s);
    return launch_quant_rows_fp8(x, rows, H, reinterpret_cast<uint8_t*>(base + q.o_q),
                                 reinterpret_cast<float*>(base + q.o_qs), s);
  }
  if (wdt == MOE_MXFP4_A4) {
    f.a_q = reinterpret_cast<const uint8_t*>(base + q.o_q);
    f.a_xs = reinterpret_cast<const uint8_t*>(base + q.o_qs);
    return launch_quant_rows_mxfp4(x, rows, H, reinterpret_cast<uint8_t*>(base + q.o_q),
                                   reinterpret_cast<uint8_t*>(base + q.o_qs), s);
  }
  return hipSuccess;
}

struct LayerPlan {
  size_t o_route = 0, o_idx = 0, o_w = 0, o_counts = 0, o_offsets = 0, o_perm_src = 0,
         o_inv_perm = 0, o_row_token = 0, o_perm_ws = 0;
  QPlan q;
  // the shared group's own tile list, for the launch that runs beside the routed experts
  size_t o_sh_tiles = 0, o_sh_ntiles = 0;
  int32_t sh_max_tiles = 0;
  // the streaming kernels' tile list of the groups moe_layer_forward_split runs beside the rest
  size_t o_cold_tiles = 0, o_cold_ntiles = 0;
  int32_t cold_max_tiles = 0;
  FfnPlan ffn;
  size_t total = 0;
};

LayerPlan plan_layer(const moe_layer_desc* d) {
  LayerPlan p;
  Carve c;
  const int32_t T = d->T, H = d->H, E = d->E, k = d->k;
  const bool shared = d->shared.w13 != nullptr;
  const int64_t rows = (int64_t)T * k;
  p.o_route = c.take(route_ws_bytes(T, H, E));
  p.o_idx = c.take(rows * sizeof(int32_t));
  p.o_w = c.take(rows * sizeof(float));
  p.o_counts = c.take(E * sizeof(int32_t));
  p.o_offsets = c.take((E + 1) * sizeof(int32_t));
  p.o_perm_src = c.take(rows * sizeof(int32_t));
  p.o_inv_perm = c.take(rows * sizeof(int32_t));
  p.o_row_token = c.take((rows + (shared ? T : 0)) * sizeof(int32_t));
  p.o_perm_ws = c.take(permute_ws_bytes(T, E));
  plan_quant(c, p.q, d->routed.dtype, T, H);
  plan_ffn(c, p.ffn, d->routed.dtype, d->act_dtype, H, d->routed.I, shared ? d->shared.I : 0,
           (int32_t)rows, E, shared ? T : 0, true);
  if (shared) {
    p.sh_max_tiles = (T + p.ffn.tile_m - 1) / p.ffn.tile_m;
    p.o_sh_tiles = c.take((size_t)(p.sh_max_tiles > 0 ? p.sh_max_tiles : 1) * sizeof(Tile));
    p.o_sh_ntiles = c.take(sizeof(int32_t));
  }
  p.cold_max_tiles = (int32_t)max_tiles(rows + (shared ? T : 0), E + 1, ffn_stream_tile_rows());
  p.o_cold_tiles = c.take((size_t)p.cold_max_tiles * sizeof(Tile));
  p.o_cold_ntiles = c.take(sizeof(int32_t));
  p.total = c.off;
  return p;
}

moe_status check_layer(const moe_layer_desc* d) {
  if (!d) return MOE_ERR_NULL;
  if (!d->w_router) return MOE_ERR_NULL;
  const bool shared = d->shared.w13 != nullptr;
  if (d->T < 0 || d->H < 1 || d->E < 1 || d->k < 1 || d->k > d->E || d->k > 16)
    return MOE_ERR_SHAPE;
  if (d->E + (shared ? 1 : 0) > 1024) return MOE_ERR_SHAPE;
  if ((int64_t)d->T * (d->k + 1) >= ((int64_t)1 << 31)) return MOE_ERR_SHAPE;
  if (d->score_fn != MOE_SOFTMAX && d->score_fn != MOE_SIGMOID) return MOE_ERR_SHAPE;
  if (!io_dt_ok(d->act_dtype) || !io_dt_ok(d->out_dtype)) return MOE_ERR_DTYPE;
  if (!act_ok(d->act_dtype, d->routed.dtype)) return MOE_ERR_DTYPE;
  if (d->routed.E != d->E) return MOE_ERR_SHAPE;
  moe_status st = check_bank(&d->routed, d->H, true);
  if (st != MOE_OK) return st;
  if (shared) {
    if (d->shared.dtype != d->routed.dtype) return MOE_ERR_DTYPE;
    if (d->shared.E != 1) return MOE_ERR_SHAPE;
    st = check_bank(&d->shared, d->H, true);
    if (st != MOE_OK) return st;
  }
  if (!al16(d->w_router) || (d->bias && !al16(d->bias))) return MOE_ERR_ALIGN;
  return MOE_OK;
}

BankView view(const moe_experts& w) {
  BankView v;
  v.w13 = w.w13;
  v.w13_scale = w.w13_scale;
  v.w2 = w.w2;
  v.w2_scale = w.w2_scale;
  v.I = w.I;
  return v;
}

FfnArgs ffn_args(const FfnPlan& p, char* ws, const moe_experts& routed, const moe_experts* shared,
                 moe_dtype act, int32_t H, const void* a, const int32_t* rowmap, void* y) {
  FfnArgs f;
  memset(&f, 0, sizeof f);
  f.wdt = routed.dtype;
  f.act_dt = act;
  f.y_dt = p.y_dt;
  f.E = routed.E;
  f.has_shared = shared != nullptr;
  f.H = H;
  f.I_max = p.I_max;
  f.bank[0] = view(routed);
  if (shared) f.bank[1] = view(*shared);
  f.a = a;
  f.a_rowmap = rowmap;
  f.y = y;
  f.tiles = reinterpret_cast<const Tile*>(ws + p.o_tiles);
  f.ntiles = reinterpret_cast<const int32_t*>(ws + p.o_ntiles);
  f.max_tiles = p.max_tiles;
  f.tile_m = p.tile_m;
  f.rows_total = p.rows_total;
  return f;
}

}  // namespace

extern "C" {

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "required pointer is NULL";
    case MOE_ERR_SHAPE: return "size out of range or not a supported multiple";
    case MOE_ERR_DTYPE: return "unsupported dtype or dtype combination";
    case MOE_ERR_ALIGN: return "pointer not aligned as required";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

const char* moe_last_hip_error(void) { return g_last_hip; }

// ------------------------------------------------------------------------- route

size_t moe_route_workspace_size(int32_t T, int32_t H, int32_t E) {
  if (T < 0 || H < 1 || E < 1) return 0;
  return route_ws_bytes(T, H, E);
}

moe_status moe_route(const void* x, moe_dtype x_dt, const void* w_router, const float* bias,
                     int32_t T, int32_t H, int32_t E, int32_t k, moe_score_fn fn,
                     float route_scale, int32_t* topk_idx, float* topk_w, float* logits, void* ws,
                     size_t ws_bytes, void* stream) {
  if (T < 0 || H < 1 || E < 1 || E > 1024 || k < 1 || k > E || k > 16 || H % 8)
    return MOE_ERR_SHAPE;
  if (fn != MOE_SOFTMAX && fn != MOE_SIGMOID) return MOE_ERR_SHAPE;
  if (!io_dt_ok(x_dt)) return MOE_ERR_DTYPE;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !topk_idx || !topk_w || !ws) return MOE_ERR_NULL;
  if (!al16(x) || !al16(w_router) || (bias && !al16(bias)) || !al16(topk_idx) || !al16(topk_w) ||
      (logits && !al16(logits)) || !al256(ws))
    return MOE_ERR_ALIGN;
  if (ws_bytes < route_ws_bytes(T, H, E)) return MOE_ERR_WORKSPACE;
  hipError_t e = launch_route(x, x_dt, w_router, bias, T, H, E, k, fn, route_scale, topk_idx,
                              topk_w, logits, ws, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_route");
}

// ----------------------------------------------------------------------- permute

size_t moe_permute_workspace_size(int32_t T, int32_t k, int32_t E) {
  (void)k;
  if (T < 0 || E < 1) return 0;
  return permute_ws_bytes(T, E);
}

moe_status moe_permute(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E, const void* x,
                       moe_dtype x_dt, int32_t H, int32_t* counts, int32_t* offsets,
                       int32_t* perm_src, int32_t* inv_perm, void* x_perm, void* ws,
                       size_t ws_bytes, void* stream) {
  if (T < 0 || E < 1 || E > 1024 || k < 1 || k > E || k > 16) return MOE_ERR_SHAPE;
  if ((int64_t)T * k >= ((int64_t)1 << 31)) return MOE_ERR_SHAPE;
  if (!counts || !offsets || !ws) return MOE_ERR_NULL;
  if (T > 0 && (!topk_idx || !perm_src || !inv_perm)) return MOE_ERR_NULL;
  if ((x == nullptr) != (x_perm == nullptr)) return MOE_ERR_NULL;
  if (x) {
    if (!io_dt_ok(x_dt)) return MOE_ERR_DTYPE;
    if (H < 1 || (H * (int64_t)dt_bytes(x_dt)) % 16) return MOE_ERR_SHAPE;
    if (!al16(x) || !al16(x_perm)) return MOE_ERR_ALIGN;
  }
  if (!al256(ws)) return MOE_ERR_ALIGN;
  if (ws_bytes < permute_ws_bytes(T, E)) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_permute_maps(topk_idx, T, k, E, counts, offsets, perm_src, inv_perm,
                                     nullptr, nullptr, nullptr, 1, 0, ws, s);
  if (e != hipSuccess) return hip_fail(e, "moe_permute");
  if (x) {
    e = launch_gather_rows(x, (int32_t)dt_bytes(x_dt), H, perm_src, k, T * k, x_perm, s);
    if (e != hipSuccess) return hip_fail(e, "moe_permute gather");
  }
  return MOE_OK;
}

// ------------------------------------------------------------------- grouped FFN


static bool plan_grouped(const moe_experts* w, moe_dtype act_dt, int32_t rows, FfnPlan* p,
                         QPlan* q, size_t* total) {
  Carve c;
  plan_quant(c, *q, w->dtype, rows, w->H);
  plan_ffn(c, *p, w->dtype, act_dt, w->H, w->I, 0, rows, w->E, 0, false);
  *total = c.off;
  return true;
}

size_t moe_grouped_ffn_workspace_size(const moe_experts* w, moe_dtype act_dt, int32_t rows) {
  if (!w || rows < 0 || w->E < 1 || w->H < 1 || w->I < 1) return 0;
  FfnPlan p;
  QPlan q;
  size_t total;
  plan_grouped(w, act_dt, rows, &p, &q, &total);
  return total;
}

moe_status moe_grouped_ffn(const moe_experts* w, const void* x_perm, moe_dtype act_dt,
                           const int32_t* offsets, int32_t rows, void* y_perm, moe_dtype y_dt,
                           void* ws, size_t ws_bytes, void* stream) {
  if (!w) return MOE_ERR_NULL;
  if (rows < 0 || (int64_t)rows * 8 >= ((int64_t)1 << 31) || w->E > 1024) return MOE_ERR_SHAPE;
  moe_status st = check_bank(w, w->H, true);
  if (st != MOE_OK) return st;
  if (!act_ok(act_dt, w->dtype) || !io_dt_ok(y_dt)) return MOE_ERR_DTYPE;
  if (!offsets || !ws) return MOE_ERR_NULL;
  if (rows > 0 && (!x_perm || !y_perm)) return MOE_ERR_NULL;
  if ((x_perm && !al16(x_perm)) || (y_perm && !al16(y_perm)) || !al256(ws)) return MOE_ERR_ALIGN;
  FfnPlan p;
  QPlan q;
  size_t total;
  plan_grouped(w, act_dt, rows, &p, &q, &total);
  if (ws_bytes < total) return MOE_ERR_WORKSPACE;
  char* base = reinterpret_cast<char*>(ws);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_tiles_from_offsets(offsets, w->E, reinterpret_cast<Tile*>(base + p.o_tiles),
                                           reinterpret_cast<int32_t*>(base + p.o_ntiles), p.tile_m, s);
  if (e != hipSuccess) return hip_fail(e, "moe_grouped_ffn tiles");
  FfnArgs f = ffn_args(p, base, *w, nullptr, act_dt, w->H, x_perm, nullptr, y_perm);
  f.y_dt = y_dt;
  e = quantise_acts(w->dtype, x_perm, rows, w->H, base, q, f, s);
  if (e != hipSuccess) return hip_fail(e, "moe_grouped_ffn quantise");
  e = launch_grouped_ffn(f, base + p.o_scratch, s);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_grouped_ffn");
}

moe_status moe_grouped_ffn_prequant(const moe_experts* w, const void* x_codes,
                                    const void* x_scales, const int32_t* offsets, int32_t rows,
                                    void* y_perm, moe_dtype y_dt, void* ws, size_t ws_bytes,
                                    void* stream) {
  if (!w) return MOE_ERR_NULL;
  if (rows < 0 || (int64_t)rows * 8 >= ((int64_t)1 << 31) || w->E > 1024) return MOE_ERR_SHAPE;
  moe_status st = check_bank(w, w->H, true);
  if (st != MOE_OK) return st;
  const bool q8 = w->dtype == MOE_FP8_E4M3 || w->dtype == MOE_INT8;
  if (!(q8 || w->dtype == MOE_MXFP4_A4) || !io_dt_ok(y_dt)) return MOE_ERR_DTYPE;
  if (!offsets || !ws) return MOE_ERR_NULL;
  if (rows > 0 && (!x_codes || !x_scales || !y_perm)) return MOE_ERR_NULL;
  if ((x_codes && !al16(x_codes)) || (x_scales && !al16(x_scales)) || (y_perm && !al16(y_perm)) ||
      !al256(ws))
    return MOE_ERR_ALIGN;
  FfnPlan p;
  QPlan q;
  size_t total;
  plan_grouped(w, MOE_BF16, rows, &p, &q, &total);
  if (ws_bytes < total) return MOE_ERR_WORKSPACE;
  char* base = reinterpret_cast<char*>(ws);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_tiles_from_offsets(offsets, w->E, reinterpret_cast<Tile*>(base + p.o_tiles),
                                           reinterpret_cast<int32_t*>(base + p.o_ntiles), p.tile_m, s);
  if (e != hipSuccess) return hip_fail(e, "moe_grouped_ffn_prequant tiles");
  // the kernels of these formats read only the codes and scales of the rows
  FfnArgs f = ffn_args(p, base, *w, nullptr, MOE_BF16, w->H, nullptr, nullptr, y_perm);
  f.y_dt = y_dt;
  f.a_q = reinterpret_cast<const uint8_t*>(x_codes);
  if (q8) f.a_qscale = reinterpret_cast<const float*>(x_scales);
  else f.a_xs = reinterpret_cast<const uint8_t*>(x_scales);
  e = launch_grouped_ffn(f, base + p.o_scratch, s);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_grouped_ffn_prequant");
}

// ----------------------------------------------------------------------- combine

moe_status moe_combine(const void* y_perm, moe_dtype y_dt, const int32_t* inv_perm,
                       const float* topk_w, int32_t T, int32_t k, int32_t H,
                       const void* shared_out, void* out, moe_dtype out_dt, void* stream) {
  if (T < 0 || k < 1 || H < 8 || H % 8 || (int64_t)T * k >= ((int64_t)1 << 31)) return MOE_ERR_SHAPE;
  if (!io_dt_ok(y_dt) || !io_dt_ok(out_dt)) return MOE_ERR_DTYPE;
  if (T == 0) return MOE_OK;
  if (!y_perm || !inv_perm || !topk_w || !out) return MOE_ERR_NULL;
  if (!al16(y_perm) || !al16(out) || (shared_out && !al16(shared_out))) return MOE_ERR_ALIGN;
  hipError_t e = launch_combine(y_perm, y_dt, inv_perm, topk_w, T, k, H, shared_out, out, out_dt,
                                (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_combine");
}

// ------------------------------------------------------------------- whole layer

moe_status moe_layer_workspace_size(const moe_layer_desc* d, size_t* bytes) {
  if (!bytes) return MOE_ERR_NULL;
  moe_status st = check_layer(d);
  if (st != MOE_OK) return st;
  *bytes = plan_layer(d).total;
  return MOE_OK;
}

// side != nullptr: the shared expert runs on `side` between the fork and join events,
// beside route, permute and the routed experts on `stream`.
struct SideStream {
  hipStream_t s;
  hipEvent_t fork, join;
};

static moe_status layer_forward(const moe_layer_desc* d, const void* x, void* out,
                                int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out,
                                float* logits_out, void* ws, size_t ws_bytes, void* stream,
                                void* const* events, const SideStream* side = nullptr) {
  moe_status st = check_layer(d);
  if (st != MOE_OK) return st;
  if (!ws || (d->T > 0 && (!x || !out))) return MOE_ERR_NULL;
  if ((x && !al16(x)) || (out && !al16(out)) || !al256(ws)) return MOE_ERR_ALIGN;
  if ((topk_idx_out && !al16(topk_idx_out)) || (topk_w_out && !al16(topk_w_out)) ||
      (counts_out && !al16(counts_out)) || (logits_out && !al16(logits_out)))
    return MOE_ERR_ALIGN;
  const LayerPlan p = plan_layer(d);
  if (ws_bytes < p.total) return MOE_ERR_WORKSPACE;
  char* base = reinterpret_cast<char*>(ws);
  hipStream_t s = (hipStream_t)stream;
  const int32_t T = d->T, k = d->k, E = d->E, H = d->H;
  const bool shared = d->shared.w13 != nullptr;
  int32_t* idx = topk_idx_out ? topk_idx_out : reinterpret_cast<int32_t*>(base + p.o_idx);
  float* w = topk_w_out ? topk_w_out : reinterpret_cast<float*>(base + p.o_w);
  int32_t* counts = counts_out ? counts_out : reinterpret_cast<int32_t*>(base + p.o_counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + p.o_offsets);
  int32_t* perm_src = reinterpret_cast<int32_t*>(base + p.o_perm_src);
  int32_t* inv_perm = reinterpret_cast<int32_t*>(base + p.o_inv_perm);
  int32_t* row_token = reinterpret_cast<int32_t*>(base + p.o_row_token);
  hipEvent_t ev[MOE_STAGE_EVENTS] = {};
  if (events)
    for (int i = 0; i < MOE_STAGE_EVENTS; ++i) ev[i] = reinterpret_cast<hipEvent_t>(events[i]);
  hipError_t e = hipSuccess;
#define MOE_MARK(i)                                                                    \
  if (events && (e = hipEventRecord(ev[i], s)) != hipSuccess)                         \
    return hip_fail(e, "moe_layer_forward event");
  const bool beside = side && shared && T > 0;
  void* y = base + p.ffn.o_y;
  FfnArgs f = ffn_args(p.ffn, base, d->routed, shared ? &d->shared : nullptr, d->act_dtype, H, x,
                       row_token, y);
  MOE_MARK(0);
  if (beside) {  // the shared launch reads the quantised activations too
    e = quantise_acts(d->routed.dtype, x, T, H, base, p.q, f, s);
    if (e != hipSuccess) return hip_fail(e, "moe_layer_forward quantise");
  }
  if (beside) {
    if ((e = hipEventRecord(side->fork, s)) != hipSuccess ||
        (e = hipStreamWaitEvent(side->s, side->fork, 0)) != hipSuccess)
      return hip_fail(e, "moe_layer_forward fork");
    Tile* sh_tiles = reinterpret_cast<Tile*>(base + p.o_sh_tiles);
    int32_t* sh_nt = reinterpret_cast<int32_t*>(base + p.o_sh_ntiles);
    e = launch_shared_group(T, k, E, p.ffn.tile_m, row_token, sh_tiles, sh_nt, side->s);
    if (e != hipSuccess) return hip_fail(e, "moe_layer_forward shared rows");
    FfnArgs fs = f;
    fs.tiles = sh_tiles;
    fs.ntiles = sh_nt;
    fs.max_tiles = p.sh_max_tiles;
    e = launch_grouped_ffn(fs, base + p.ffn.o_scratch, side->s);
    if (e != hipSuccess) return hip_fail(e, "moe_layer_forward shared ffn");
    if ((e = hipEventRecord(side->join, side->s)) != hipSuccess)
      return hip_fail(e, "moe_layer_forward join");
  }
  e = launch_route(x, d->act_dtype, d->w_router, d->bias, T, H, E, k, d->score_fn,
                              d->route_scale, idx, w, logits_out, base + p.o_route, s);
  if (e != hipSuccess) return hip_fail(e, "moe_layer_forward route");
  MOE_MARK(1);
  e = launch_permute_maps(idx, T, k, E, counts, offsets, perm_src, inv_perm, row_token,
                          reinterpret_cast<Tile*>(base + p.ffn.o_tiles),
                          reinterpret_cast<int32_t*>(base + p.ffn.o_ntiles), p.ffn.tile_m,
                          shared && !beside ? 1 : 0, base + p.o_perm_ws, s);
  if (e != hipSuccess) return hip_fail(e, "moe_layer_forward permute");
  if (!beside) {
    e = quantise_acts(d->routed.dtype, x, T, H, base, p.q, f, s);
    if (e != hipSuccess) return hip_fail(e, "moe_layer_forward quantise");
  }
  MOE_MARK(2);
  if (beside) f.max_tiles = p.ffn.max_tiles - p.sh_max_tiles;  // routed groups only
  e = launch_grouped_ffn(f, base + p.ffn.o_scratch, s, events ? ev[3] : nullptr);
  if (e != hipSuccess) return hip_fail(e, "moe_layer_forward grouped_ffn");
  if (beside && (e = hipStreamWaitEvent(s, side->join, 0)) != hipSuccess)
    return hip_fail(e, "moe_layer_forward join");
  MOE_MARK(4);
  const void* ysh = shared ? reinterpret_cast<const char*>(y) +
                                 (size_t)T * k * H * dt_bytes(p.ffn.y_dt)
                           : nullptr;
  e = launch_combine(y, p.ffn.y_dt, inv_perm, w, T, k, H, ysh, out, d->out_dtype, s);
  if (e != hipSuccess) return hip_fail(e, "moe_layer_forward combine");
  MOE_MARK(5);
#undef MOE_MARK
  return MOE_OK;
}

moe_status moe_layer_forward(const moe_layer_desc* d, const void* x, void* out,
                             int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out,
                             float* logits_out, void* ws, size_t ws_bytes, void* stream) {
  return layer_forward(d, x, out, topk_idx_out, topk_w_out, counts_out, logits_out, ws, ws_bytes,
                       stream, nullptr);
}

moe_status moe_layer_forward_overlap(const moe_layer_desc* d, const void* x, void* out,
                                     int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out,
                                     float* logits_out, void* ws, size_t ws_bytes, void* stream,
                                     void* side_stream, void* fork_event, void* join_event) {
  if (!fork_event || !join_event) return MOE_ERR_NULL;
  const SideStream side{(hipStream_t)side_stream, (hipEvent_t)fork_event, (hipEvent_t)join_event};
  return layer_forward(d, x, out, topk_idx_out, topk_w_out, counts_out, logits_out, ws, ws_bytes,
                       stream, nullptr, &side);
}

moe_status moe_layer_forward_split(const moe_layer_desc* d, const void* x, void* out,
                                   int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out,
                                   float* logits_out, void* ws, size_t ws_bytes, void* stream,
                                   void* cold_stream, void* fork_event, void* join_event,
                                   int32_t cold_rows_max) {
  moe_status st = check_layer(d);
  if (st != MOE_OK) return st;
  if (d->routed.dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (cold_rows_max < 0) return MOE_ERR_SHAPE;
  if (!fork_event || !join_event || !ws || (d->T > 0 && (!x || !out))) return MOE_ERR_NULL;
  if ((x && !al16(x)) || (out && !al16(out)) || !al256(ws)) return MOE_ERR_ALIGN;
  if ((topk_idx_out && !al16(topk_idx_out)) || (topk_w_out && !al16(topk_w_out)) ||
      (counts_out && !al16(counts_out)) || (logits_out && !al16(logits_out)))
    return MOE_ERR_ALIGN;
  const LayerPlan p = plan_layer(d);
  if (ws_bytes < p.total) return MOE_ERR_WORKSPACE;
  const int32_t T = d->T, k = d->k, E = d->E, H = d->H;
  if (T == 0) return MOE_OK;
  char* base = reinterpret_cast<char*>(ws);
  hipStream_t s = (hipStream_t)stream, sc = (hipStream_t)cold_stream;
  hipEvent_t fork = (hipEvent_t)fork_event, join = (hipEvent_t)join_event;
  const bool shared = d->shared.w13 != nullptr;
  int32_t* idx = topk_idx_out ? topk_idx_out : reinterpret_cast<int32_t*>(base + p.o_idx);
  float* w = topk_w_out ? topk_w_out : reinterpret_cast<float*>(base + p.o_w);
  int32_t* counts = counts_out ? counts_out : reinterpret_cast<int32_t*>(base + p.o_counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + p.o_offsets);
  int32_t* inv_perm = reinterpret_cast<int32_t*>(base + p.o_inv_perm);
  int32_t* row_token = reinterpret_cast<int32_t*>(base + p.o_row_token);
  hipError_t e = launch_route(x, d->act_dtype, d->w_router, d->bias, T, H, E, k, d->score_fn,
                              d->route_scale, idx, w, logits_out, base + p.o_route, s);
  if (e != hipSuccess) return hip_fail(e, "moe_layer_forward_split route");
  e = launch_permute_maps(idx, T, k, E, counts, offsets,
                          reinterpret_cast<int32_t*>(base + p.o_perm_src), inv_perm, row_token,
                          nullptr, nullptr, p.ffn.tile_m, shared ? 1 : 0, base + p.o_perm_ws, s);
  if (e != hipSuccess) return hip_fail(e, "moe_layer_forward_split permute");
  const int32_t tm_cold = ffn_stream_tile_rows();
  Tile* hot_tiles = reinterpret_cast<Tile*>(base + p.ffn.o_tiles);
  int32_t* hot_n = reinterpret_cast<int32_t*>(base + p.ffn.o_ntiles);
  Tile* cold_tiles = reinterpret_cast<Tile*>(base + p.o_cold_tiles);
  int32_t* cold_n = reinterpret_cast<int32_t*>(base + p.o_cold_ntiles);
  e = launch_split_tiles(offsets, E, T, k, shared ? 1 : 0, cold_rows_max, p.ffn.tile_m, hot_tiles,
                         hot_n, tm_cold, cold_tiles, cold_n, s);
  if (e != hipSuccess) return hip_fail(e, "moe_layer_forward_split tiles");
  void* y = base + p.ffn.o_y;
  FfnArgs f = ffn_args(p.ffn, base, d->routed, shared ? &d->shared : nullptr, d->act_dtype, H, x,
                       row_token, y);
  // cold groups: streaming kernels on the side stream, between the fork and join events; at
  // most ceil(cold_rows_max / tm_cold) tiles a group
  FfnArgs fc = f;
  fc.tiles = cold_tiles;
  fc.ntiles = cold_n;
  fc.tile_m = tm_cold;
  const int64_t per_group = ((int64_t)cold_rows_max + tm_cold - 1) / tm_cold;
  const int64_t cold_bound = per_group * (E + (shared ? 1 : 0));
  fc.max_tiles = (int32_t)(cold_bound < p.cold_max_tiles ? cold_bound : p.cold_max_tiles);
  if ((e = hipEventRecord(fork, s)) != hipSuccess || (e = hipStreamWaitEvent(sc, fork, 0)) != hipSuccess)
    return hip_fail(e, "moe_layer_forward_split fork");
  e = launch_grouped_ffn(fc, base + p.ffn.o_scratch, sc);
  if (e != hipSuccess) return hip_fail(e, "moe_layer_forward_split cold ffn");
  if ((e = hipEventRecord(join, sc)) != hipSuccess) return hip_fail(e, "moe_layer_forward_split join");
  // hot groups: the kernels the layer picks for this batch, on the main stream
  e = launch_grouped_ffn(f, base + p.ffn.o_scratch, s);
  if (e != hipSuccess) return hip_fail(e, "moe_layer_forward_split hot ffn");
  if ((e = hipStreamWaitEvent(s, join, 0)) != hipSuccess)
    return hip_fail(e, "moe_layer_forward_split join");
  const void* ysh = shared ? reinterpret_cast<const char*>(y) + (size_t)T * k * H * dt_bytes(p.ffn.y_dt)
                           : nullptr;
  e = launch_combine(y, p.ffn.y_dt, inv_perm, w, T, k, H, ysh, out, d->out_dtype, s);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_layer_forward_split combine");
}

moe_status moe_layer_forward_timed(const moe_layer_desc* d, const void* x, void* out,
                                   int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out,
                                   float* logits_out, void* ws, size_t ws_bytes, void* stream,
                                   void* const* events) {
  if (!events) return MOE_ERR_NULL;
  for (int i = 0; i < MOE_STAGE_EVENTS; ++i)
    if (!events[i]) return MOE_ERR_NULL;
  return layer_forward(d, x, out, topk_idx_out, topk_w_out, counts_out, logits_out, ws, ws_bytes,
                       stream, events);
}

// ---------------------------------------------------- no-allocation layer forward

// The workspace of moe_layer_forward_noalloc: one copy on every GPU the library runs on,
// held until the process ends. In host code this name is a host-side stand-in, not a
// device address: the address of each GPU's copy comes from hipGetSymbolAddress, looked
// up once per device with that device current, and only that address is ever passed on.
static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the stream's device (looked up on the first call there).
hipError_t scratch_on(hipStream_t s, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (s) {
    hipDevice_t sd;
    if ((e = hipStreamGetDevice(s, &sd)) != hipSuccess) return e;
    dev = (int)sd;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (!p || ((uintptr_t)p & 255u)) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}
}  // namespace

moe_status moe_layer_forward_noalloc(const moe_layer_desc* d, const void* x, void* out,
                                     int32_t* topk_idx_out, float* topk_w_out,
                                     int32_t* counts_out, float* logits_out, void* stream) {
  size_t need = 0;
  moe_status st = moe_layer_workspace_size(d, &need);
  if (st != MOE_OK) return st;
  if (need > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  hipError_t e = scratch_on((hipStream_t)stream, &ws);
  if (e != hipSuccess) return hip_fail(e, "moe_layer_forward_noalloc scratch address");
  return layer_forward(d, x, out, topk_idx_out, topk_w_out, counts_out, logits_out, ws,
                       MOE_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

// ------------------------------------------------------------- pre-routed rows

static size_t plan_rows(const moe_experts* w, moe_dtype act_dt, int32_t rows, size_t o[6],
                        FfnPlan* fp, QPlan* qp) {
  Carve c;
  plan_quant(c, *qp, w->dtype, rows, w->H);
  o[0] = c.take(w->E * sizeof(int32_t));             // counts
  o[1] = c.take((w->E + 1) * sizeof(int32_t));       // offsets
  o[2] = c.take((size_t)rows * sizeof(int32_t));     // perm_src
  o[3] = c.take((size_t)rows * sizeof(int32_t));     // inv_perm
  o[4] = c.take((size_t)rows * sizeof(int32_t));     // row_token
  o[5] = c.take(permute_ws_bytes(rows, w->E));
  plan_ffn(c, *fp, w->dtype, act_dt, w->H, w->I, 0, rows, w->E, 0, true);
  return c.off;
}

size_t moe_rows_workspace_size(const moe_experts* w, moe_dtype act_dt, int32_t rows) {
  if (!w || rows < 0 || w->E < 1 || w->H < 1 || w->I < 1) return 0;
  size_t o[6];
  FfnPlan fp;
  QPlan qp;
  return plan_rows(w, act_dt, rows, o, &fp, &qp);
}

static moe_status rows_forward(const moe_experts* w, const void* x, moe_dtype act_dt,
                               const int32_t* row_expert, const float* row_w, int32_t rows,
                               void* out, moe_dtype out_dt, void* ws, size_t ws_bytes,
                               void* stream, void* const* events) {
  if (!w) return MOE_ERR_NULL;
  if (rows < 0 || (int64_t)rows * 2 >= ((int64_t)1 << 31) || w->E > 1024) return MOE_ERR_SHAPE;
  moe_status st = check_bank(w, w->H, true);
  if (st != MOE_OK) return st;
  if (!act_ok(act_dt, w->dtype) || !io_dt_ok(out_dt)) return MOE_ERR_DTYPE;
  if (!ws) return MOE_ERR_NULL;
  if (rows > 0 && (!x || !row_expert || !row_w || !out)) return MOE_ERR_NULL;
  if ((x && !al16(x)) || (out && !al16(out)) || !al256(ws)) return MOE_ERR_ALIGN;
  size_t o[6];
  FfnPlan p;
  QPlan qp;
  size_t total = plan_rows(w, act_dt, rows, o, &p, &qp);
  if (ws_bytes < total) return MOE_ERR_WORKSPACE;
  char* base = reinterpret_cast<char*>(ws);
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t ev[MOE_STAGE_EVENTS] = {};
  if (events)
    for (int i = 0; i < MOE_STAGE_EVENTS; ++i) ev[i] = reinterpret_cast<hipEvent_t>(events[i]);
  hipError_t e = hipSuccess;
  // the stage layout of moe_layer_forward_timed; there is no route stage here
#define MOE_MARK(i)                                                                    \
  if (events && (e = hipEventRecord(ev[i], s)) != hipSuccess)                         \
    return hip_fail(e, "moe_rows_forward event");
  MOE_MARK(0);
  MOE_MARK(1);
  int32_t* inv_perm = reinterpret_cast<int32_t*>(base + o[3]);
  int32_t* row_token = reinterpret_cast<int32_t*>(base + o[4]);
  e = launch_permute_maps(row_expert, rows, 1, w->E, reinterpret_cast<int32_t*>(base + o[0]),
                                     reinterpret_cast<int32_t*>(base + o[1]),
                                     reinterpret_cast<int32_t*>(base + o[2]), inv_perm, row_token,
                                     reinterpret_cast<Tile*>(base + p.o_tiles),
                                     reinterpret_cast<int32_t*>(base + p.o_ntiles), p.tile_m, 0,
                                     base + o[5], s);
  if (e != hipSuccess) return hip_fail(e, "moe_rows_forward permute");
  void* y = base + p.o_y;
  FfnArgs f = ffn_args(p, base, *w, nullptr, act_dt, w->H, x, row_token, y);
  e = quantise_acts(w->dtype, x, rows, w->H, base, qp, f, s);
  if (e != hipSuccess) return hip_fail(e, "moe_rows_forward quantise");
  MOE_MARK(2);
  e = launch_grouped_ffn(f, base + p.o_scratch, s, events ? ev[3] : nullptr);
  if (e != hipSuccess) return hip_fail(e, "moe_rows_forward grouped_ffn");
  MOE_MARK(4);
  e = launch_combine(y, p.y_dt, inv_perm, row_w, rows, 1, w->H, nullptr, out, out_dt, s);
  if (e != hipSuccess) return hip_fail(e, "moe_rows_forward combine");
  MOE_MARK(5);
#undef MOE_MARK
  return MOE_OK;
}

moe_status moe_rows_forward(const moe_experts* w, const void* x, moe_dtype act_dt,
                            const int32_t* row_expert, const float* row_w, int32_t rows,
                            void* out, moe_dtype out_dt, void* ws, size_t ws_bytes, void* stream) {
  return rows_forward(w, x, act_dt, row_expert, row_w, rows, out, out_dt, ws, ws_bytes, stream,
                      nullptr);
}

moe_status moe_rows_forward_timed(const moe_experts* w, const void* x, moe_dtype act_dt,
                                  const int32_t* row_expert, const float* row_w, int32_t rows,
                                  void* out, moe_dtype out_dt, void* ws, size_t ws_bytes,
                                  void* stream, void* const* events) {
  if (!events) return MOE_ERR_NULL;
  return rows_forward(w, x, act_dt, row_expert, row_w, rows, out, out_dt, ws, ws_bytes, stream,
                      events);
}

// --------------------------------------------------------------- fp8 quantiser

moe_status moe_quantize_fp8(const void* x, int32_t n, int32_t H, uint8_t* q, float* q_scale,
                            void* stream) {
  if (n < 0 || H < 128 || H % 128) return MOE_ERR_SHAPE;
  if (n == 0) return MOE_OK;
  if (!x || !q || !q_scale) return MOE_ERR_NULL;
  if (!al16(x) || !al16(q) || !al16(q_scale)) return MOE_ERR_ALIGN;
  hipError_t e = launch_quant_rows_fp8(x, n, H, q, q_scale, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_quantize_fp8");
}

// ------------------------------------------------------------- INT8 quantiser

moe_status moe_quantize_int8(const void* x, int32_t n, int32_t H, int8_t* q, float* q_scale,
                             void* stream) {
  if (n < 0 || H < 128 || H % 128) return MOE_ERR_SHAPE;
  if (n == 0) return MOE_OK;
  if (!x || !q || !q_scale) return MOE_ERR_NULL;
  if (!al16(x) || !al16(q) || !al16(q_scale)) return MOE_ERR_ALIGN;
  hipError_t e = launch_quant_rows_int8(x, n, H, q, q_scale, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_quantize_int8");
}

// ------------------------------------------------------------- bias balancing

moe_status moe_bias_update(const int32_t* counts, int32_t E, float u, float* bias,
                           void* stream) {
  if (E < 1 || E > 1024) return MOE_ERR_SHAPE;
  if (!__builtin_isfinite(u)) return MOE_ERR_SHAPE;
  if (!counts || !bias) return MOE_ERR_NULL;
  if (!al16(counts) || !al16(bias)) return MOE_ERR_ALIGN;
  hipError_t e = launch_bias_update(counts, E, u, bias, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_bias_update");
}

// ------------------------------------------------------------- MXFP4 quantiser

moe_status moe_quantize_mxfp4(const void* x, int32_t n, int32_t H, uint8_t* q, uint8_t* q_scale,
                              void* stream) {
  if (n < 0 || H < 32 || H % 32) return MOE_ERR_SHAPE;
  if (n == 0) return MOE_OK;
  if (!x || !q || !q_scale) return MOE_ERR_NULL;
  if (!al16(x) || !al16(q)) return MOE_ERR_ALIGN;
  hipError_t e = launch_quant_rows_mxfp4(x, n, H, q, q_scale, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_quantize_mxfp4");
}

// ------------------------------------------------------------- measurement probes

moe_status moe_probe_hbm_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (bytes == 0 || bytes % 16 || bytes > ((size_t)1 << 40)) return MOE_ERR_SHAPE;
  if (!buf || !sink) return MOE_ERR_NULL;
  if (!al16(buf)) return MOE_ERR_ALIGN;
  hipError_t e = launch_probe_read(buf, (int64_t)bytes, sink, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_probe_hbm_read");
}

moe_status moe_probe_mfma(moe_dtype dtype, int64_t iters, uint32_t* sink, double* flops,
                          void* stream) {
  if (dtype != MOE_BF16 && dtype != MOE_FP8_E4M3 && dtype != MOE_INT8 && dtype != MOE_MXFP4_A4)
    return MOE_ERR_DTYPE;
  if (iters < 1 || iters > (1 << 30)) return MOE_ERR_SHAPE;
  if (!sink || !flops) return MOE_ERR_NULL;
  hipError_t e = launch_probe_mfma(dtype, iters, sink, flops, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_probe_mfma");
}

}  // extern "C"
