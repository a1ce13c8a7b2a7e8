"""CPU oracle of the sparse MoE feed-forward layer, in float64 numpy.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package's smoke check and the
benchmark's CPU-baseline leg may import this module. The GPU library neither
imports it nor shares any code with it; it is the slow, plain statement of what
the layer computes, against which the HIP kernels are checked.

What is computed, and where it comes from:
  * The layer skeleton -- router logits, top-k selection with renormalised
    weights, dispatch of each token to its chosen experts, a weighted sum of the
    expert outputs, plus an always-active shared expert -- follows the moe_ffn
    pseudocode in "Decoding Trillion-Parameter MoE LLMs: Sparse Architecture and
    Agentic Intelligence" (section "Routing: Top-K Experts Plus a Shared Expert").
    Each token goes to k distinct experts (the WideEP claim card on DeepSeek R1,
    "Context Before" paragraph).
  * A per-expert bias that steers selection without entering the weights is the
    "auxiliary-loss-free bias routing" named in the roadmap of "Chapter 7:
    Serving Mega-MoE at Scale". The pages give no formula; the reading used is
    key = score + bias for selection, weights from the unbiased scores.
  * The update of that bias from the batch's expert loads is a reading too (the pages
    name the technique, not its rule); see bias_update.
  * The expert FFN is SwiGLU, and fp8 / MXFP4 weights with fp8 re-quantisation
    of the SwiGLU output follow the FP8/FP4 grouped GEMM with fused SwiGLU and
    re-quantisation in "GC-MoE: Overlapping Expert-Parallel Token Dispatch with
    FP8/FP4 Grouped GEMM via CUDA Green Contexts" (key_changes, fourth item).
  * INT8 weights and activations (W8A8) follow section 3.1 of "Trillion-Parameter LLM
    Architecture Explained and Cost-Efficient Inference in Practice"; the recipe (symmetric,
    fp32 block scales amax/127) is a reading, see quantise_rows_int8.
  * Readings where the pages are silent (sigmoid or softmax scoring, the 2.5
    scale, fp64 accumulation of the router, tie-breaking, block-scale layouts)
    are stated at each function.

Inputs are storage-format arrays (fp32 values, bf16 bit patterns as uint16,
E4M3FN codes, packed E2M1 nibbles with E8M0 scales); the oracle decodes them to
float64 itself. Parity of the layer outputs on the named workloads is pinned only
through the checks in the test suite (brute force, closed forms, library
routines, invariants): the pages print no worked example.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------- codecs

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64: the bf16 value is the fp32 with these top 16 bits."""
    u = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def f32_to_f64(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, np.float32).astype(np.float64)


def _e4m3_values(c: np.ndarray) -> np.ndarray:
    """OCP 8-bit floating point E4M3 (the 'FN' variant: bias 7, no infinities,
    S.1111.111 is NaN). Normal: (1 + m/8) * 2^(e-7); subnormal (e = 0): m/8 * 2^-6."""
    c = np.asarray(c, np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7))
    out = s * mag
    return np.where((e == 15) & ((c & 7) == 7), np.nan, out)


# the value of every E4M3 code, from the definition above: decoding is a table look-up
_E4M3_VALUES = _e4m3_values(np.arange(256))


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """E4M3FN codes -> float64 values (see _e4m3_values)."""
    return _E4M3_VALUES[np.asarray(codes, np.uint8)]


def _e2m1_values(n: np.ndarray) -> np.ndarray:
    """OCP MX E2M1 element (bias 1): normal (1 + m/2) * 2^(e-1); subnormal m * 0.5."""
    n = np.asarray(n, np.int64) & 0xF
    s = np.where(n & 0x8, -1.0, 1.0)
    e = (n >> 1) & 0x3
    m = (n & 0x1).astype(np.float64)
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e.astype(np.float64) - 1))
    return s * mag


_E2M1_VALUES = _e2m1_values(np.arange(16))


def e2m1_to_f64(nibbles: np.ndarray) -> np.ndarray:
    """E2M1 nibbles (the low 4 bits of each byte) -> float64 values (see _e2m1_values)."""
    return _E2M1_VALUES[np.asarray(nibbles, np.uint8) & 0xF]


def e8m0_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP MX E8M0 scale: 2^(code - 127); code 255 is NaN."""
    c = np.asarray(codes, np.uint8).astype(np.float64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def _e4m3_grid() -> np.ndarray:
    """The 127 non-negative finite E4M3FN values, indexed by their code 0..126."""
    return e4m3_to_f64(np.arange(127, dtype=np.uint8))


def encode_e4m3_rne_sat(v32: np.ndarray) -> np.ndarray:
    """Nearest E4M3FN code to each fp32 value, ties to the even code, magnitudes
    beyond 448 clamped to 448 (saturating conversion). Written as the definition:
    the nearest point of the finite value grid."""
    v = np.asarray(v32, np.float32).astype(np.float64)
    grid = _e4m3_grid()
    a = np.minimum(np.abs(v), grid[-1])
    hi = np.clip(np.searchsorted(grid, a, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    dlo = a - grid[lo]
    dhi = grid[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == grid[hi], hi, code).astype(np.uint8)
    return np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)


def quantise_rows_e4m3(v32: np.ndarray, block: int = 128):
    """Per-row, per-`block`-column fp8 quantisation of fp32 activations.

    Reading (the pages name FP8 with re-quantisation but fix no recipe): for each
    1 x 128 block, scale s = fp32(amax / 448) (s = 1 for an all-zero block) and
    code q = E4M3(fp32(v / s)) with round-to-nearest-even and saturation; the
    dequantised value is q * s. Decisions are taken in fp32.
    Returns (codes uint8 [R, C], scales f32 [R, C/block], dequantised f64 [R, C]).
    """
    v = np.asarray(v32, np.float32)
    R, C = v.shape
    vb = v.reshape(R, C // block, block)
    amax = np.abs(vb).max(axis=2)
    s = np.where(amax == 0, np.float32(1.0), (amax / np.float32(448.0)).astype(np.float32))
    s = s.astype(np.float32)
    scaled = (vb / s[:, :, None]).astype(np.float32)
    codes = encode_e4m3_rne_sat(scaled).reshape(R, C)
    deq = (e4m3_to_f64(codes).reshape(R, C // block, block) * s[:, :, None].astype(np.float64))
    return codes, s, deq.reshape(R, C)


def quantise_rows_int8(v32: np.ndarray, block: int = 128):
    """Per-row, per-`block`-column INT8 quantisation of fp32 values (the W8A8 path).

    Reading ("Trillion-Parameter LLM Architecture Explained and Cost-Efficient Inference in
    Practice", section 3.1 names W8A8 -- weights and activations as INT8 on INT8 matrix
    units -- but fixes no recipe): symmetric INT8 with the block structure of the FP8
    path. For each 1 x 128 block, scale s = fp32(amax / 127) (s = 1 for an all-zero block)
    and code q = round-half-to-even(fp32(v / s)), clamped to [-127, 127]; the dequantised
    value is q * s. Decisions are taken in fp32.
    Returns (codes int8 [R, C], scales f32 [R, C/block], dequantised f64 [R, C]).
    """
    v = np.asarray(v32, np.float32)
    R, C = v.shape
    vb = v.reshape(R, C // block, block)
    amax = np.abs(vb).max(axis=2)
    s = np.where(amax == 0, np.float32(1.0), (amax / np.float32(127.0)).astype(np.float32))
    s = s.astype(np.float32)
    scaled = (vb / s[:, :, None]).astype(np.float32)
    codes = np.clip(np.rint(scaled), -127, 127).astype(np.int8).reshape(R, C)
    deq = codes.astype(np.float64).reshape(R, C // block, block) * s[:, :, None].astype(np.float64)
    return codes, s, deq.reshape(R, C)


def _e2m1_grid() -> np.ndarray:
    """The 8 non-negative E2M1 values, indexed by their code 0..7."""
    return e2m1_to_f64(np.arange(8, dtype=np.uint8))


def encode_e2m1_rne_sat(v: np.ndarray) -> np.ndarray:
    """Nearest E2M1 code (a nibble) to each value, ties to the even code, magnitudes beyond
    6 clamped to 6: the nearest point of the value grid, written as the definition."""
    v = np.asarray(v, np.float64)
    grid = _e2m1_grid()
    a = np.minimum(np.abs(v), grid[-1])
    hi = np.clip(np.searchsorted(grid, a, side="left"), 0, 7)
    lo = np.clip(hi - 1, 0, 7)
    dlo = a - grid[lo]
    dhi = grid[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == grid[hi], hi, code).astype(np.uint8)
    return np.where(np.signbit(v), code | 0x8, code).astype(np.uint8)


def quantise_rows_mxfp4(v32: np.ndarray, block: int = 32):
    """Per-row, per-32-column MXFP4 quantisation of fp32 values (the W4A4 path).

    Reading, from the OCP MX format the FP4 grouped GEMM of GC-MoE uses (the pages fix no
    recipe): the block's shared scale is 2^e with e = floor(log2(amax)) - 2, where 2 is the
    exponent of E2M1's largest value 6 (e clamped to [-127, 127]; e = 0 for an all-zero
    block); each element's code is E2M1(v / 2^e), round to nearest even, saturating at 6.
    Returns (codes uint8 nibbles [R, C], E8M0 scale codes uint8 [R, C/block], dequantised
    f64 [R, C]).
    """
    v = np.asarray(v32, np.float32).astype(np.float64)
    R, C = v.shape
    vb = v.reshape(R, C // block, block)
    amax = np.abs(vb).max(axis=2)
    _, ex = np.frexp(amax)                    # amax = m * 2^ex, m in [0.5, 1)
    e = np.where(amax == 0, 0, np.clip(ex - 1 - 2, -127, 127)).astype(np.int64)
    scale = np.exp2(e.astype(np.float64))
    codes = encode_e2m1_rne_sat(vb / scale[:, :, None]).reshape(R, C)
    deq = (e2m1_to_f64(codes).reshape(R, C // block, block) * scale[:, :, None]).reshape(R, C)
    return codes, (e + 127).astype(np.uint8), deq


def decode_matrix(fmt: str, part: dict) -> np.ndarray:
    """One expert matrix [R, C] in storage format -> float64.

    fp8: E4M3 codes times the fp32 scale of their 128 x 128 block.
    int8: INT8 codes times the fp32 scale of their 128 x 128 block.
    mxfp4: E2M1 nibbles (element 2i in the low nibble of byte i) times 2^(e8m0 - 127)
    of their 32-element block along C.
    """
    w = part["w"]
    if fmt == "f32":
        return f32_to_f64(w)
    if fmt == "bf16":
        return bf16_to_f64(w)
    if fmt in ("fp8", "int8"):
        s = np.asarray(part["scale"], np.float32).astype(np.float64)
        R, C = w.shape
        codes = e4m3_to_f64(w) if fmt == "fp8" else np.asarray(w, np.int8).astype(np.float64)
        v = codes.reshape(R // 128, 128, C // 128, 128)
        return (v * s[:, None, :, None]).reshape(R, C)
    if fmt in ("mxfp4", "mxfp4a4"):
        p = np.asarray(w, np.uint8)
        R = p.shape[0]
        C = p.shape[1] * 2
        el = np.empty((R, C), np.uint8)
        el[:, 0::2] = p & 0xF
        el[:, 1::2] = p >> 4
        sc = e8m0_to_f64(part["scale"])
        return (e2m1_to_f64(el).reshape(R, C // 32, 32) * sc[:, :, None]).reshape(R, C)
    raise ValueError(fmt)


def decode_act(fmt: str, x: np.ndarray) -> np.ndarray:
    return bf16_to_f64(x) if fmt == "bf16" else f32_to_f64(x)


# ----------------------------------------------------------------------------- routing

def router_logits(x64: np.ndarray, wr64: np.ndarray) -> np.ndarray:
    """Router scores of each token for each expert (moe_ffn's gate(x)).
    Reading: the dot products are formed in float64 and rounded once to fp32."""
    return (x64 @ wr64.T).astype(np.float32)


def scores(logits32: np.ndarray, fn: str) -> np.ndarray:
    """Score per (token, expert) in float64 from the fp32 logits.
    sigmoid: 1 / (1 + e^-l).  softmax: e^(l - max) / sum_e e^(l - max) over all E
    (moe_ffn's topk_softmax, read as softmax over all experts then renormalised)."""
    l = logits32.astype(np.float64)
    if fn == "sigmoid":
        return 1.0 / (1.0 + np.exp(-l))
    if fn == "softmax":
        z = np.exp(l - l.max(axis=1, keepdims=True))
        return z / z.sum(axis=1, keepdims=True)
    raise ValueError(fn)


def selection_keys(s64: np.ndarray, bias) -> np.ndarray:
    """Selection key in fp32: fp32(score), plus the per-expert bias as one fp32 add.
    The bias enters only here (auxiliary-loss-free bias routing)."""
    s32 = s64.astype(np.float32)
    if bias is None:
        return s32
    return (s32 + np.asarray(bias, np.float32)[None, :]).astype(np.float32)


def select_topk(keys32: np.ndarray, k: int) -> np.ndarray:
    """The k experts with the largest keys per token, as expert ids in ascending order.

    Order: larger key first; equal keys (with -0 == +0) go to the lower expert index;
    NaN ranks below every number (NaNs among themselves by lower index). This order is
    total, so the chosen set is unique.
    """
    T, E = keys32.shape
    kk = keys32.astype(np.float64)
    isnan = np.isnan(kk)
    filled = np.where(isnan, 0.0, kk)
    idx = np.broadcast_to(np.arange(E), (T, E))
    out = np.empty((T, k), np.int32)
    for t in range(T):
        order = np.lexsort((idx[t], -filled[t], isnan[t]))
        out[t] = np.sort(order[:k])
    return out


def routing_weights(s64: np.ndarray, topk_idx: np.ndarray, scale: float) -> np.ndarray:
    """Weights of the chosen experts: their unbiased scores renormalised to sum to one,
    times `scale` (moe_ffn's 'normalize weights'; the scale is a stated reading)."""
    sel = np.take_along_axis(s64, topk_idx.astype(np.int64), axis=1)
    return scale * sel / sel.sum(axis=1, keepdims=True)


def route(x64, wr64, bias, k: int, fn: str, scale: float):
    logits = router_logits(x64, wr64)
    s64 = scores(logits, fn)
    keys = selection_keys(s64, bias)
    idx = select_topk(keys, k)
    w = routing_weights(s64, idx, scale)
    return {"logits": logits, "scores": s64, "keys": keys, "topk_idx": idx, "topk_w": w}


# ----------------------------------------------------------------------------- dispatch

def permutation(topk_idx: np.ndarray, E: int):
    """Dispatch of (token, slot) assignments into contiguous per-expert groups.

    counts[e] = number of tokens that chose e; offsets = exclusive prefix sum
    (offsets[E] = T*k); rows are ordered by expert, then by token (stable), so the
    map is unique. perm_src[r] = t*k + j for the assignment held by row r, and
    inv_perm[t*k + j] = r.
    """
    T, k = topk_idx.shape
    e_flat = topk_idx.reshape(-1).astype(np.int64)
    t_flat = np.repeat(np.arange(T, dtype=np.int64), k)
    counts = np.bincount(e_flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    order = np.lexsort((t_flat, e_flat))           # by expert, then token
    perm_src = order.astype(np.int32)              # flat assignment index t*k + j
    inv_perm = np.empty(T * k, np.int32)
    inv_perm[order] = np.arange(T * k, dtype=np.int32)
    return counts, offsets.astype(np.int32), perm_src, inv_perm


# ----------------------------------------------------------------------------- balancing

def bias_update(bias, counts, u: float) -> np.ndarray:
    """One step of auxiliary-loss-free balancing of the selection bias.

    The pages name the technique ("auxiliary-loss-free bias routing", roadmap of
    "Chapter 7: Serving Mega-MoE at Scale") and its purpose -- keep the router from
    piling traffic on a few experts without an auxiliary loss term ("Decoding
    Trillion-Parameter MoE LLMs", sections "Routing: Top-K Experts Plus a Shared Expert"
    and "Engineering Reality: Sparse Activation Is Not Free") -- but print no rule. The
    reading used: an expert's load is the number of tokens routed to it in the batch
    (`counts`), the mean load is sum(counts) / E, and

        b_e <- b_e + u * sign(mean - load_e)

    so an under-loaded expert's key is raised by u, an over-loaded one's lowered by u, and
    one exactly at the mean gets b + u * 0. The step u is an fp32 number, like the bias
    (the rule is written for a stored fp32 bias and step). Evaluated in float64; the result
    is stored in fp32, the format the router reads the bias in.
    """
    c = np.asarray(counts, np.float64)
    mean = c.sum() / c.size
    b64 = np.asarray(bias, np.float32).astype(np.float64)
    u64 = np.float64(np.float32(u))
    return (b64 + u64 * np.sign(mean - c)).astype(np.float32)


# ----------------------------------------------------------------------------- experts

def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + e^-z)."""
    return z / (1.0 + np.exp(-z))


def expert_ffn(a64: np.ndarray, w13_64: np.ndarray, w2_64: np.ndarray, requant_h=False):
    """SwiGLU expert: g = a Wg^T, u = a Wu^T, h = SiLU(g) * u, y = h W2^T, where W13's
    first I rows are Wg and the next I rows Wu. With requant_h (True or "fp8"), h is
    re-quantised to E4M3 per 1x128 block (from its fp32 value) before the down
    projection, as the fused SwiGLU + re-quantisation of the fp8 grouped GEMM does; with
    "mxfp4", to MXFP4 per 1x32 block (the W4A4 path); with "int8", to INT8 per 1x128 block
    (the W8A8 path)."""
    I = w13_64.shape[0] // 2
    g = a64 @ w13_64[:I].T
    u = a64 @ w13_64[I:].T
    h = silu(g) * u
    if requant_h == "mxfp4":
        _, _, h = quantise_rows_mxfp4(h.astype(np.float32))
    elif requant_h == "int8":
        _, _, h = quantise_rows_int8(h.astype(np.float32))
    elif requant_h:
        _, _, h = quantise_rows_e4m3(h.astype(np.float32))
    return h @ w2_64.T


def expert_weights(bank, e: int):
    """Decode expert e of a bank (an object with fmt, w13(e), w2(e)) to float64."""
    return decode_matrix(bank.fmt, bank.w13(e)), decode_matrix(bank.fmt, bank.w2(e))


# ----------------------------------------------------------------------------- layer

def layer_forward(prob, tokens=None, with_routing: bool = True, workers: int = 1):
    """The whole layer on the host for the listed tokens (default: all).

    Routing, counts and the permutation always cover all T tokens (they are global);
    expert outputs are computed only for the listed tokens, one expert at a time, so
    a sample of a large layer only decodes the experts that sample touches.
    out[t] = sum_j w[t,j] * FFN_{e_j}(x_t) + FFN_shared(x_t); pre-routed rows
    (no router) give out[r] = w_r * FFN_{e_r}(x_r).
    workers > 1 decodes and evaluates that many experts at once on threads; their
    contributions are still added in ascending expert order, so the result is the same.
    """
    cfg = prob.cfg
    T = cfg.T
    tokens = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    x64 = decode_act(cfg.act, prob.x)
    res = {}
    if cfg.routed:
        r = route(x64, decode_act(cfg.act, prob.wr), prob.bias, cfg.k, cfg.score, cfg.scale)
        res.update(r)
        topk_idx, topk_w = r["topk_idx"], r["topk_w"]
    else:
        topk_idx = np.asarray(prob.topk_idx, np.int32)
        topk_w = np.asarray(prob.topk_w, np.float32).astype(np.float64)
        res["topk_idx"], res["topk_w"] = topk_idx, topk_w
    counts, offsets, perm_src, inv_perm = permutation(topk_idx, cfg.E)
    res.update(counts=counts, offsets=offsets, perm_src=perm_src, inv_perm=inv_perm)

    fp8 = cfg.wdt == "fp8"
    a4 = cfg.wdt == "mxfp4a4"
    i8 = cfg.wdt == "int8"
    requant = "mxfp4" if a4 else ("int8" if i8 else fp8)
    xs = x64[tokens]
    if fp8:
        # activations enter the expert GEMMs quantised per 1x128 block (from bf16/fp32)
        _, _, a = quantise_rows_e4m3(xs.astype(np.float32))
    elif i8:
        # W8A8: activations quantised to INT8 per 1x128 block
        _, _, a = quantise_rows_int8(xs.astype(np.float32))
    elif a4:
        # W4A4: activations quantised to MXFP4 per 1x32 block
        _, _, a = quantise_rows_mxfp4(xs.astype(np.float32))
    else:
        a = xs
    out = np.zeros((len(tokens), cfg.H), np.float64)
    sel = topk_idx[tokens]
    wsel = topk_w[tokens]

    def contribution(e):
        rows, slots = np.nonzero(sel == e)
        w13, w2 = expert_weights(prob.routed, int(e))
        return rows, wsel[rows, slots][:, None] * expert_ffn(a[rows], w13, w2, requant_h=requant)

    experts = np.unique(sel)
    if workers > 1:
        from concurrent.futures import ThreadPoolExecutor

        with ThreadPoolExecutor(workers) as pool:
            parts = pool.map(contribution, experts)   # yields in ascending expert order
            for rows, y in parts:
                out[rows] += y
    else:
        for e in experts:
            rows, y = contribution(e)
            out[rows] += y
    if prob.shared is not None:
        w13, w2 = expert_weights(prob.shared, 0)
        out += expert_ffn(a, w13, w2, requant_h=requant)
    res["tokens"] = tokens
    res["out"] = out
    return res


def rel_err(got: np.ndarray, want64: np.ndarray, rms: float | None = None) -> float:
    """max |got - want| / RMS(want): the comparison metric for layer outputs."""
    want64 = np.asarray(want64, np.float64)
    if rms is None:
        rms = float(np.sqrt(np.mean(want64 ** 2)))
    return float(np.max(np.abs(np.asarray(got, np.float64) - want64)) / rms)


def combine(y64: np.ndarray, inv_perm: np.ndarray, topk_w64: np.ndarray, shared64=None):
    """moe_ffn's accumulation: out[t] = sum_j w[t,j] * y[inv_perm[t*k+j]] (+ shared[t])."""
    T, k = topk_w64.shape
    rows = y64[np.asarray(inv_perm, np.int64).reshape(T, k)]          # [T, k, H]
    out = np.einsum("tk,tkh->th", topk_w64, rows)
    if shared64 is not None:
        out = out + shared64
    return out
