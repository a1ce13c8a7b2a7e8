/* moe.h -- C ABI of the sparse MoE feed-forward layer for AMD Instinct MI355X (gfx950).
 *
 * The layer (moe_ffn in "Decoding Trillion-Parameter MoE LLMs: Sparse Architecture and
 * Agentic Intelligence", section "Routing: Top-K Experts Plus a Shared Expert"):
 *
 *   logits = x Wr^T                                   router scores          (moe_route)
 *   S_t    = top-k experts of score(logits_t) + bias   selection only
 *   w_t    = scale * score_S / sum(score_S)            renormalised weights
 *   rows   = tokens regrouped by expert                dispatch               (moe_permute)
 *   y_r    = SwiGLU_e(x_r)                             grouped expert FFN     (moe_grouped_ffn)
 *   out_t  = sum_j w_tj y_(t,j) + SwiGLU_shared(x_t)   weighted combine       (moe_combine)
 *
 * moe_layer_forward runs all of it. Every step runs in the library's own HIP kernels.
 *
 * Conventions (all entry points):
 *  - Tensor arguments are DEVICE pointers (HBM), row-major, the last dimension
 *    contiguous. Descriptor structs and scalars are passed from the host. The caller
 *    allocates and owns every buffer, including the workspace; the library allocates
 *    nothing and keeps no device state between calls (the one exception: the static
 *    workspace of moe_layer_forward_noalloc, which holds no result between calls).
 *  - Calls are asynchronous: they only enqueue kernels on `stream` (a hipStream_t; NULL
 *    is the default stream) and never synchronise or copy to the host, so they may be
 *    captured into a HIP graph. Group sizes stay on the device.
 *  - All arguments are validated on the host before anything is enqueued. On an error
 *    nothing is launched and outputs are untouched. Launch failures return MOE_ERR_HIP
 *    (text from moe_last_hip_error). Faults inside kernels surface at the caller's next
 *    synchronisation. No C++ exception crosses this boundary; the library never prints.
 *  - Shapes are int32; internal addressing is 64-bit.
 *  - Tensor pointers must be 16-byte aligned; the workspace 256-byte aligned.
 *  - Calls on different streams may run concurrently if their buffers do not overlap.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,      /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,     /* a size is out of range or not a multiple the format needs */
  MOE_ERR_DTYPE = 3,     /* unsupported dtype or dtype combination */
  MOE_ERR_ALIGN = 4,     /* a pointer is not aligned as required */
  MOE_ERR_WORKSPACE = 5, /* ws_bytes is smaller than the *_workspace_size result */
  MOE_ERR_HIP = 6        /* a HIP launch failed */
} moe_status;

typedef enum {
  MOE_F32 = 0,      /* IEEE binary32 */
  MOE_BF16 = 1,     /* bfloat16 */
  MOE_FP8_E4M3 = 2, /* OCP E4M3FN codes, with fp32 block scales */
  MOE_MXFP4 = 3,    /* OCP MX E2M1 pairs per byte (element 2i in the low nibble),
                       with E8M0 scales per 32 elements along the contiguous dimension */
  MOE_MXFP4_A4 = 4, /* expert weights only: stored as MOE_MXFP4, and the layer quantises the
                       activations (and the SwiGLU output) to MXFP4 too, per 1 x 32 block:
                       scale 2^(floor(log2 amax) - 2) (1 for a zero block), codes E2M1 with
                       round to nearest even, saturating at 6 -- both operands of the expert
                       GEMMs are then FP4 (W4A4) */
  MOE_INT8 = 5      /* expert weights only: symmetric INT8 codes (two's complement) with fp32
                       block scales; the layer quantises the activations (and the SwiGLU
                       output) to INT8 per 1 x 128 block: scale amax / 127 (1 for a zero
                       block), codes round-to-nearest-even of x / scale clamped to +-127 --
                       both operands of the expert GEMMs are then INT8 (W8A8) */
} moe_dtype;

typedef enum {
  MOE_SOFTMAX = 0, /* softmax over all E logits */
  MOE_SIGMOID = 1  /* logistic sigmoid of each logit */
} moe_score_fn;

/* One bank of SwiGLU experts (E = 1 for a shared expert).
 *   w13 [E, 2I, H]: rows [0, I) are the gate projection, rows [I, 2I) the up projection.
 *   w2  [E, H, I] : the down projection.
 * FP8_E4M3: codes as above; w13_scale f32 [E, 2I/128, H/128], w2_scale f32 [E, H/128, I/128]
 *           (one scale per 128 x 128 block; value = code * scale). H, I multiples of 128.
 * MXFP4:    w13 bytes [E, 2I, H/2], w2 bytes [E, H, I/2]; w13_scale u8 [E, 2I, H/32],
 *           w2_scale u8 [E, H, I/32] (value = e2m1 * 2^(scale - 127)). H, I multiples of 128.
 *           A scale byte of 0xFF (NaN in the OCP format) makes its block non-finite: the
 *           batched (tiled) kernels decode it as +Inf (zero codes give NaN, others +-Inf),
 *           the decode-sized ones as NaN.
 * MXFP4_A4: the MXFP4 layout; activations BF16 in, quantised inside. H, I multiples of 128.
 * INT8:     w13 int8 [E, 2I, H], w2 int8 [E, H, I]; w13_scale f32 [E, 2I/128, H/128],
 *           w2_scale f32 [E, H/128, I/128] (value = code * scale; the W8A8 weights of
 *           section 3.1 of "Trillion-Parameter LLM Architecture Explained and
 *           Cost-Efficient Inference in Practice"). Activations BF16 in, quantised inside.
 *           H, I multiples of 128.
 * F32/BF16: no scales (NULL). H, I multiples of 8 (multiples of 64 run on the matrix cores;
 *           other multiples of 8 on plain fp32 dot products with h kept in fp32).
 * The fp8 and MXFP4 expert formats are the FP8/FP4 grouped GEMM inputs of "GC-MoE:
 * Overlapping Expert-Parallel Token Dispatch with FP8/FP4 Grouped GEMM via CUDA Green
 * Contexts" (key_changes, fourth item); block shapes are this library's choice. */
typedef struct {
  moe_dtype dtype;
  const void* w13;
  const void* w13_scale;
  const void* w2;
  const void* w2_scale;
  int32_t E, H, I;
} moe_experts;

/* ---------------------------------------------------------------------------- routing */

/* Bytes of workspace moe_route needs for these sizes (pure host function). */
size_t moe_route_workspace_size(int32_t T, int32_t H, int32_t E);

/* Router scores, selection and routing weights for T tokens (moe_ffn's gate and
 * topk_softmax; bias routing from the roadmap of "Chapter 7: Serving Mega-MoE at Scale").
 *   x        [T, H] activations, x_dt F32 or BF16.
 *   w_router [E, H] router weights, same dtype as x.
 *   bias     [E] f32 selection bias, or NULL for none.
 *   logits   [T, E] f32 = fp32(sum_h x w_r), accumulated in fp64; optional (NULL).
 *   score    sigmoid: 1/(1+e^-l); softmax over all E.  Computed in fp64 from the fp32 logit.
 *   key      fp32(score) + bias[e] (fp32). The k largest keys win; equal keys go to the
 *            lower expert id; NaN ranks lowest. Exactly k distinct experts per token.
 *   topk_idx [T, k] int32 chosen expert ids in ascending order.
 *   topk_w   [T, k] f32 = route_scale * score_e / sum over chosen score (unbiased scores).
 * With bf16 inputs, logits == NULL, H % 64 == 0 and T >= 512 the selection is first made
 * from bf16 matrix-core dot products with a proven error bound and kept where that bound
 * separates the chosen keys from the rest (the weights then come from exact fp64 dot
 * products of the chosen experts); every other token goes through the fp64 path. The
 * expert ids are the same either way; weights agree to fp32 rounding.
 * Limits: 1 <= k <= min(E, 16), E <= 1024, T >= 0, H >= 1 and H % 8 == 0. */
moe_status moe_route(const void* x, moe_dtype x_dt, const void* w_router, const float* bias,
                     int32_t T, int32_t H, int32_t E, int32_t k, moe_score_fn fn,
                     float route_scale, int32_t* topk_idx, float* topk_w, float* logits,
                     void* ws, size_t ws_bytes, void* stream);

/* --------------------------------------------------------------------------- dispatch */

size_t moe_permute_workspace_size(int32_t T, int32_t k, int32_t E);

/* Regroups the T*k (token, slot) assignments into contiguous per-expert rows, ordered by
 * expert id and, inside an expert, by token index (moe_ffn's dispatch, which is an
 * all-to-all between GPUs in an expert-parallel deployment and a row gather on one GPU).
 *   topk_idx [T, k] int32, each row k distinct ids in [0, E).
 *   counts   [E] int32 rows per expert;  offsets [E+1] int32 exclusive prefix sum.
 *   perm_src [T*k] int32: row r holds assignment perm_src[r] = t*k + j.
 *   inv_perm [T*k] int32: assignment t*k + j sits in row inv_perm[t*k + j].
 *   x        [T, H] (x_dt F32/BF16) or NULL for maps only; x_perm [T*k, H] receives
 *            x_perm[r] = x[perm_src[r] / k] (NULL iff x is NULL).
 * Limits: 1 <= k <= min(E,16), E <= 1024, T*k < 2^31. Ids outside [0, E) are undefined
 * behaviour of the caller (they are not checked on the device). */
moe_status moe_permute(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E, const void* x,
                       moe_dtype x_dt, int32_t H, int32_t* counts, int32_t* offsets,
                       int32_t* perm_src, int32_t* inv_perm, void* x_perm, void* ws,
                       size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ grouped expert FFN */

size_t moe_grouped_ffn_workspace_size(const moe_experts* w, moe_dtype act_dt, int32_t rows);

/* SwiGLU FFN of each expert e on its rows [offsets[e], offsets[e+1]) of x_perm, as one
 * grouped GEMM pair: h = SiLU(x Wg^T) * (x Wu^T), y = h W2^T (moe_ffn's e(x); SwiGLU and
 * the fused epilogue follow GC-MoE's grouped GEMM with fused SwiGLU).
 *   w        expert bank (see moe_experts), w->E groups.
 *   x_perm   [rows, H] act_dt: F32 with F32 weights; BF16 with every other format.
 *            With FP8_E4M3 weights, rows are quantised inside to E4M3 per 1 x 128 block
 *            (scale = amax/448) and h is re-quantised the same way before the down GEMM;
 *            with INT8 weights, to INT8 per 1 x 128 block (scale = amax/127), likewise;
 *            with MXFP4_A4 weights, to MXFP4 per 1 x 32 block.
 *   offsets  [E+1] int32 device array, offsets[0] = 0, non-decreasing, offsets[E] = rows.
 *   y_perm   [rows, H] y_dt (F32 or BF16; F32 keeps the expert outputs unrounded until the
 *            combine, as moe_layer_forward does).
 * Limits: rows >= 0, rows < 2^31 / 8. */
moe_status moe_grouped_ffn(const moe_experts* w, const void* x_perm, moe_dtype act_dt,
                           const int32_t* offsets, int32_t rows, void* y_perm, moe_dtype y_dt,
                           void* ws, size_t ws_bytes, void* stream);

/* moe_grouped_ffn on rows that the caller has already quantised, for FP8_E4M3, INT8 and
 * MXFP4_A4 banks (the low-precision grouped GEMM of GC-MoE, key_changes, fourth item, takes
 * its activations as codes plus block scales). Codes and scales are in the layout that
 * moe_quantize_fp8, moe_quantize_int8 and moe_quantize_mxfp4 write:
 *   FP8_E4M3  x_codes [rows, H] E4M3 bytes,      x_scales [rows, H/128] f32;
 *   INT8      x_codes [rows, H] int8,            x_scales [rows, H/128] f32;
 *   MXFP4_A4  x_codes [rows, H/2] E2M1 pairs,    x_scales [rows, H/32] E8M0 bytes.
 * Both 16-byte aligned. offsets, y_perm, y_dt and the limits are moe_grouped_ffn's; the
 * workspace is moe_grouped_ffn_workspace_size(w, MOE_BF16, rows) bytes. h is re-quantised
 * inside exactly as in moe_grouped_ffn, so with the codes and scales of the matching
 * moe_quantize_* call on bf16 rows x the output is bit-identical to
 * moe_grouped_ffn(w, x, MOE_BF16, ...). Scales are used as given (not checked on the
 * device). MOE_ERR_DTYPE for any other bank format. */
moe_status moe_grouped_ffn_prequant(const moe_experts* w, const void* x_codes,
                                    const void* x_scales, const int32_t* offsets, int32_t rows,
                                    void* y_perm, moe_dtype y_dt, void* ws, size_t ws_bytes,
                                    void* stream);

/* ------------------------------------------------------------------------------ combine */

/* out[t] = sum_j topk_w[t,j] * y_perm[inv_perm[t*k+j]] + shared_out[t]   (moe_ffn's
 * weighted sum plus the always-active shared expert), summed in fp32 in slot order and
 * rounded once to out_dt.
 *   y_perm [T*k, H] y_dt; shared_out [T, H] y_dt or NULL; out [T, H] out_dt (F32 / BF16). */
moe_status moe_combine(const void* y_perm, moe_dtype y_dt, const int32_t* inv_perm,
                       const float* topk_w, int32_t T, int32_t k, int32_t H,
                       const void* shared_out, void* out, moe_dtype out_dt, void* stream);

/* -------------------------------------------------------------------------- whole layer */

typedef struct {
  int32_t T, H, E, k;
  moe_score_fn score_fn;
  float route_scale;
  moe_dtype act_dtype; /* x: F32 or BF16 */
  moe_dtype out_dtype; /* out: F32 or BF16 */
  const void* w_router; /* [E, H], act_dtype */
  const float* bias;    /* [E] selection bias, or NULL */
  moe_experts routed;   /* E experts */
  moe_experts shared;   /* shared.w13 == NULL: no shared expert; else E = 1, same dtype and H */
} moe_layer_desc;

/* Bytes of workspace moe_layer_forward needs for this descriptor (pure host function). */
moe_status moe_layer_workspace_size(const moe_layer_desc* d, size_t* bytes);

/* The whole layer: route, permute, grouped SwiGLU FFN of the routed experts and the
 * shared expert (as one more group), weighted combine.
 *   x [T, H] act_dtype; out [T, H] out_dtype.
 *   Optional outputs (NULL to skip): topk_idx_out [T, k] int32, topk_w_out [T, k] f32,
 *   counts_out [E] int32, logits_out [T, E] f32. */
moe_status moe_layer_forward(const moe_layer_desc* d, const void* x, void* out,
                             int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out,
                             float* logits_out, void* ws, size_t ws_bytes, void* stream);

/* moe_layer_forward with the always-on shared expert run beside the rest: its grouped FFN
 * goes on side_stream, forked after `stream`'s earlier work and joined back before the
 * combine, so it overlaps the router, the permutation and the routed experts (the
 * single-GPU counterpart of the concurrent shared-expert node in the CUDA-graph design of
 * "GC-MoE: Overlapping Expert-Parallel Token Dispatch with FP8/FP4 Grouped GEMM via CUDA
 * Green Contexts", key_changes, second item). Same arguments, checks, workspace size and
 * results (bit for bit) as moe_layer_forward, plus:
 *   side_stream  a hipStream_t other than `stream` (NULL is the default stream);
 *   fork_event, join_event  hipEvent_t created by the caller (timing may be disabled);
 *                MOE_ERR_NULL if either is NULL.
 * Only events are recorded and waited on, so the pair of streams can be captured into a
 * HIP graph from `stream`. Without a shared expert this is moe_layer_forward. */
moe_status moe_layer_forward_overlap(const moe_layer_desc* d, const void* x, void* out,
                                     int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out,
                                     float* logits_out, void* ws, size_t ws_bytes, void* stream,
                                     void* side_stream, void* fork_event, void* join_event);

/* moe_layer_forward with the routed and shared groups split by size over two streams: groups
 * with at most cold_rows_max rows in this batch (expert weights to stream, few rows to
 * multiply: HBM-bound work) run the grouped FFN's streaming kernels on cold_stream, the others
 * (many rows: MFMA-bound work) the kernels moe_layer_forward picks for the batch, on `stream`
 * -- so that the two kinds of tiles overlap, each on the compute units its stream may use
 * (the single-GPU counterpart of the green-context partition and the concurrent
 * dispatch/GEMM graph of "GC-MoE: Overlapping Expert-Parallel Token Dispatch with FP8/FP4
 * Grouped GEMM via CUDA Green Contexts", key_changes, first and second items; a caller can
 * create the two streams with disjoint CU masks, hipExtStreamCreateWithCUMask).
 * Same arguments, checks and workspace size as moe_layer_forward, plus:
 *   cold_stream  a hipStream_t other than `stream`;
 *   fork_event, join_event  caller hipEvent_t (MOE_ERR_NULL if NULL): cold_stream waits for
 *                `stream` after the permutation, `stream` for cold_stream before the combine;
 *   cold_rows_max  >= 0 (MOE_ERR_SHAPE otherwise); 0 sends nothing to cold_stream.
 * BF16 expert banks only (MOE_ERR_DTYPE otherwise). Routing is identical to
 * moe_layer_forward's; the cold groups' outputs come from the streaming kernels instead of
 * the tiled ones (the same arithmetic in another summation order). Only events are recorded
 * and waited on, so the pair of streams can be captured into a HIP graph. */
moe_status moe_layer_forward_split(const moe_layer_desc* d, const void* x, void* out,
                                   int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out,
                                   float* logits_out, void* ws, size_t ws_bytes, void* stream,
                                   void* cold_stream, void* fork_event, void* join_event,
                                   int32_t cold_rows_max);

/* moe_layer_forward with stage timing: `events` points to MOE_STAGE_EVENTS hipEvent_t
 * handles created by the caller (hipEventCreate); they are recorded on `stream` at the
 * stage boundaries  [0] route [1] permute [2] gate/up+SwiGLU [3] down [4] combine [5],
 * so hipEventElapsedTime(events[i], events[i+1]) is the time of stage i. The kernels and
 * their launch configurations are exactly those of moe_layer_forward. */
#define MOE_STAGE_EVENTS 6
moe_status moe_layer_forward_timed(const moe_layer_desc* d, const void* x, void* out,
                                   int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out,
                                   float* logits_out, void* ws, size_t ws_bytes, void* stream,
                                   void* const* events);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): moe_layer_forward with the library's own
 * static workspace instead of a caller's. Same descriptor, checks, kernels, launch
 * configurations and results (bit for bit) as moe_layer_forward.
 *   The workspace is a device array of MOE_NOALLOC_SCRATCH_BYTES held by the library on
 *   every GPU it runs on until the process ends; its device address is looked up once per
 *   device (on the first call there, with the stream's device made current for the lookup).
 *   Nothing is allocated and nothing in it needs clearing between calls: the kernels write
 *   every byte they read.
 *   MOE_ERR_WORKSPACE (before any HIP call) if moe_layer_workspace_size(d) exceeds
 *   MOE_NOALLOC_SCRATCH_BYTES: 64 MiB takes decode-sized batches, e.g. up to about 190
 *   tokens of a 7168-wide, 256-expert, top-8 bf16 layer with a shared expert (128 tokens:
 *   41 MiB); larger batches need moe_layer_forward and a workspace.
 *   Calls on one GPU share the array: calls that may overlap in time on one GPU (different
 *   streams, or threads without ordering) race on it and must not be issued.
 *   MOE_ERR_HIP if the device address cannot be obtained. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_layer_forward_noalloc(const moe_layer_desc* d, const void* x, void* out,
                                     int32_t* topk_idx_out, float* topk_w_out,
                                     int32_t* counts_out, float* logits_out, void* stream);

/* Pre-routed rows (one GPU's share under expert parallelism, after the dispatch exchange):
 * each of `rows` received rows carries one local expert id and one weight.
 *   out[r] = row_w[r] * SwiGLU_{row_expert[r]}(x[r]).
 * Runs permute (k = 1), the grouped FFN and combine.  x, out [rows, H] BF16 or F32. */
size_t moe_rows_workspace_size(const moe_experts* w, moe_dtype act_dt, int32_t rows);
moe_status moe_rows_forward(const moe_experts* w, const void* x, moe_dtype act_dt,
                            const int32_t* row_expert, const float* row_w, int32_t rows,
                            void* out, moe_dtype out_dt, void* ws, size_t ws_bytes, void* stream);

/* moe_rows_forward with stage timing, in the event layout of moe_layer_forward_timed
 * (events [0] and [1] are recorded together: there is no route stage). MOE_ERR_NULL if
 * events is NULL; otherwise the same checks, kernels and launch configurations as
 * moe_rows_forward. */
moe_status moe_rows_forward_timed(const moe_experts* w, const void* x, moe_dtype act_dt,
                                  const int32_t* row_expert, const float* row_w, int32_t rows,
                                  void* out, moe_dtype out_dt, void* ws, size_t ws_bytes,
                                  void* stream, void* const* events);

/* Per 1 x 128 block fp8 quantisation of activation rows, as the fp8 expert path applies it
 * to its inputs (the FP8 grouped GEMM inputs of GC-MoE, key_changes, fourth item):
 * scale = fp32(amax / 448) per block of 128 consecutive elements of a row (1 for an
 * all-zero block); code = E4M3FN(fp32(x / scale)), round to nearest even, saturating.
 *   x [n, H] BF16; q [n, H] u8 codes; q_scale [n, H/128] f32. H a multiple of 128. */
moe_status moe_quantize_fp8(const void* x, int32_t n, int32_t H, uint8_t* q, float* q_scale,
                            void* stream);

/* Per 1 x 128 block INT8 quantisation of activation rows, as the W8A8 expert path
 * (MOE_INT8) applies it to its inputs and to the SwiGLU output: scale = fp32(amax / 127) per
 * block of 128 consecutive elements of a row (1 for an all-zero block); code = round to
 * nearest even of fp32(x / scale), clamped to [-127, 127].
 *   x [n, H] BF16; q [n, H] int8 codes; q_scale [n, H/128] f32. H a multiple of 128. */
moe_status moe_quantize_int8(const void* x, int32_t n, int32_t H, int8_t* q, float* q_scale,
                             void* stream);

/* ---------------------------------------------------------------- bias balancing */

/* One step of auxiliary-loss-free balancing of the selection bias (the bias routing named
 * in the roadmap of "Chapter 7: Serving Mega-MoE at Scale"; the pages give no update rule,
 * and the one implemented is the plainest reading of the name):
 *     bias[e] <- bias[e] + u * sign(mean - counts[e]),   mean = sum(counts) / E,
 * i.e. +u for an expert that received fewer than the mean number of tokens in the batch,
 * -u for one that received more, unchanged at exactly the mean. The sign is taken in exact
 * integer arithmetic and the bias moves by one fp32 add, so the result is deterministic.
 *   counts [E] int32 routed tokens per expert (moe_permute's counts, or moe_layer_forward's
 *          counts_out); values are used as given (not checked on the device).
 *   bias   [E] f32, updated in place (the bias moe_route and moe_layer_forward read).
 *   u      step size; any finite float.
 * Limits: 1 <= E <= 1024. MOE_ERR_SHAPE for E out of range or a non-finite u. One
 * single-workgroup kernel; stream-ordered after the call that wrote counts. */
moe_status moe_bias_update(const int32_t* counts, int32_t E, float u, float* bias,
                           void* stream);

/* Per 1 x 32 block MXFP4 quantisation of activation rows, as the W4A4 expert path
 * (MOE_MXFP4_A4) applies it to its inputs and to the SwiGLU output: e = floor(log2(amax))
 * - 2 clamped to [-127, 127] (0 for an all-zero block), scale code e + 127, element codes
 * E2M1(x * 2^-e) rounded to nearest even and saturated at 6 (the OCP MX rule for the FP4
 * operands of the GC-MoE grouped GEMM, key_changes, fourth item).
 *   x [n, H] BF16; q [n, H/2] bytes (element 2i in the low nibble of byte i);
 *   q_scale [n, H/32] E8M0 bytes. H a multiple of 32. Non-finite inputs give unspecified
 *   codes. */
moe_status moe_quantize_mxfp4(const void* x, int32_t n, int32_t H, uint8_t* q, uint8_t* q_scale,
                              void* stream);

/* ---------------------------------------------------------------- measurement probes */

/* Not part of the layer: two kernels that measure the device's achievable rates, so that a
 * benchmark can state a kernel's fraction of a measured peak beside the datasheet one.
 *
 * moe_probe_hbm_read reads `bytes` of device memory at `buf` once, with non-temporal 16-B
 * loads: each wavefront streams its own contiguous chunk, 1 KB per instruction, sixteen
 * instructions in flight, two 256-thread workgroups a CU. bytes: a positive multiple of
 * 16; buf 16-byte aligned. `sink` (device, 4 bytes, caller-owned) is written only if the
 * XOR of all data read equals a fixed mark, which keeps the loads from being dropped. Time
 * the call with events on `stream`. MOE_ERR_SHAPE for bytes out of range. */
moe_status moe_probe_hbm_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* moe_probe_mfma runs four wavefronts a SIMD on every CU, each issuing `iters` rounds of
 * eight independent dense MFMAs on register operands: MOE_BF16 v_mfma_f32_16x16x32_bf16,
 * MOE_FP8_E4M3 v_mfma_scale_f32_16x16x128_f8f6f4 (unit scales), MOE_INT8
 * v_mfma_i32_16x16x64_i8, MOE_MXFP4_A4 the same scaled instruction with both operands E2M1.
 * *flops (host) receives the operations the launch executes (2 per multiply-add). sink as
 * above. MOE_ERR_DTYPE for another dtype, MOE_ERR_SHAPE for iters outside [1, 2^30]. */
moe_status moe_probe_mfma(moe_dtype dtype, int64_t iters, uint32_t* sink, double* flops,
                          void* stream);

const char* moe_status_str(moe_status s);
const char* moe_last_hip_error(void); /* thread-local text of the last MOE_ERR_HIP */

#ifdef __cplusplus
}
#endif
#endif
