"""Python binding of libmoe.so, the MI355X (gfx950) sparse MoE layer library.

Argument marshalling only: every function here passes device pointers and sizes of torch
tensors to the C ABI declared in include/moe.h, with the same names. All computation runs
in the library's HIP kernels; torch provides device memory and the current stream. There
is no fallback: if libmoe.so is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch  # loads the HIP runtime that libmoe.so then binds to

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

# enums of moe.h
MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_ALIGN, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(7)
MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_MXFP4, MOE_MXFP4_A4, MOE_INT8 = range(6)
MOE_SOFTMAX, MOE_SIGMOID = range(2)

DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3, "mxfp4": MOE_MXFP4,
          "mxfp4a4": MOE_MXFP4_A4, "int8": MOE_INT8}
SCORES = {"softmax": MOE_SOFTMAX, "sigmoid": MOE_SIGMOID}


class MoEError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = f"{what}: {lib().moe_status_str(status).decode()}"
        if status == MOE_ERR_HIP:
            msg += " -- " + lib().moe_last_hip_error().decode()
        super().__init__(msg)
        self.status = status


class moe_experts(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("w13", ctypes.c_void_p), ("w13_scale", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p), ("E", ctypes.c_int32),
                ("H", ctypes.c_int32), ("I", ctypes.c_int32)]


class moe_layer_desc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("score_fn", ctypes.c_int), ("route_scale", ctypes.c_float),
                ("act_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
                ("w_router", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("routed", moe_experts), ("shared", moe_experts)]


_lib = None
EXPORTS = ["moe_route_workspace_size", "moe_route", "moe_permute_workspace_size", "moe_permute",
           "moe_grouped_ffn_workspace_size", "moe_grouped_ffn", "moe_grouped_ffn_prequant",
           "moe_combine",
           "moe_layer_workspace_size", "moe_layer_forward", "moe_layer_forward_timed",
           "moe_layer_forward_overlap", "moe_layer_forward_noalloc", "moe_layer_forward_split",
           "moe_rows_workspace_size",
           "moe_rows_forward", "moe_rows_forward_timed", "moe_quantize_fp8", "moe_quantize_mxfp4", "moe_quantize_int8", "moe_bias_update",
           "moe_probe_hbm_read", "moe_probe_mfma", "moe_status_str",
           "moe_last_hip_error"]


def lib():
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    i32, sz, vp, f32, ci = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float, ctypes.c_int
    P = ctypes.POINTER
    L.moe_route_workspace_size.argtypes = [i32, i32, i32]
    L.moe_route_workspace_size.restype = sz
    L.moe_route.argtypes = [vp, ci, vp, vp, i32, i32, i32, i32, ci, f32, vp, vp, vp, vp, sz, vp]
    L.moe_permute_workspace_size.argtypes = [i32, i32, i32]
    L.moe_permute_workspace_size.restype = sz
    L.moe_permute.argtypes = [vp, i32, i32, i32, vp, ci, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_grouped_ffn_workspace_size.argtypes = [P(moe_experts), ci, i32]
    L.moe_grouped_ffn_workspace_size.restype = sz
    L.moe_grouped_ffn.argtypes = [P(moe_experts), vp, ci, vp, i32, vp, ci, vp, sz, vp]
    L.moe_grouped_ffn_prequant.argtypes = [P(moe_experts), vp, vp, vp, i32, vp, ci, vp, sz, vp]
    L.moe_combine.argtypes = [vp, ci, vp, vp, i32, i32, i32, vp, vp, ci, vp]
    L.moe_layer_workspace_size.argtypes = [P(moe_layer_desc), P(sz)]
    L.moe_layer_forward.argtypes = [P(moe_layer_desc), vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_layer_forward_timed.argtypes = [P(moe_layer_desc), vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                          P(vp)]
    L.moe_layer_forward_overlap.argtypes = [P(moe_layer_desc), vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                            vp, vp, vp]
    L.moe_layer_forward_noalloc.argtypes = [P(moe_layer_desc), vp, vp, vp, vp, vp, vp, vp]
    L.moe_layer_forward_split.argtypes = [P(moe_layer_desc), vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                          vp, vp, vp, i32]
    L.moe_rows_workspace_size.argtypes = [P(moe_experts), ci, i32]
    L.moe_rows_workspace_size.restype = sz
    L.moe_rows_forward.argtypes = [P(moe_experts), vp, ci, vp, vp, i32, vp, ci, vp, sz, vp]
    L.moe_rows_forward_timed.argtypes = [P(moe_experts), vp, ci, vp, vp, i32, vp, ci, vp, sz, vp,
                                         P(vp)]
    for f in ("moe_route", "moe_permute", "moe_grouped_ffn", "moe_grouped_ffn_prequant", "moe_combine", "moe_layer_workspace_size",
              "moe_layer_forward", "moe_layer_forward_timed", "moe_layer_forward_overlap",
              "moe_layer_forward_noalloc", "moe_layer_forward_split",
              "moe_rows_forward",
              "moe_rows_forward_timed"):
        getattr(L, f).restype = ci
    L.moe_quantize_fp8.argtypes = [vp, i32, i32, vp, vp, vp]
    L.moe_quantize_fp8.restype = ci
    L.moe_quantize_int8.argtypes = [vp, i32, i32, vp, vp, vp]
    L.moe_quantize_int8.restype = ci
    L.moe_quantize_mxfp4.argtypes = [vp, i32, i32, vp, vp, vp]
    L.moe_quantize_mxfp4.restype = ci
    L.moe_bias_update.argtypes = [vp, i32, f32, vp, vp]
    L.moe_bias_update.restype = ci
    L.moe_probe_hbm_read.argtypes = [vp, sz, vp, vp]
    L.moe_probe_hbm_read.restype = ci
    L.moe_probe_mfma.argtypes = [ci, ctypes.c_int64, vp, P(ctypes.c_double), vp]
    L.moe_probe_mfma.restype = ci
    L.moe_status_str.argtypes = [ci]
    L.moe_status_str.restype = ctypes.c_char_p
    L.moe_last_hip_error.argtypes = []
    L.moe_last_hip_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _act_dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"activation dtype {t.dtype} is not float32 or bfloat16")


def _check(st: int, what: str):
    if st != MOE_OK:
        raise MoEError(st, what)


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


@dataclass
class Experts:
    """A bank of SwiGLU experts in HBM (w13 [E,2I,H], w2 [E,H,I]; see moe.h for fp8/MXFP4)."""
    fmt: str
    E: int
    H: int
    I: int
    w13: torch.Tensor
    w2: torch.Tensor
    w13_scale: Optional[torch.Tensor] = None
    w2_scale: Optional[torch.Tensor] = None

    @classmethod
    def from_bank(cls, bank) -> "Experts":
        """From any object with the same fields (fmt, E, H, I, w13, w2, w13_scale, w2_scale),
        e.g. a bank of the seeded workload generator."""
        return cls(bank.fmt, bank.E, bank.H, bank.I, bank.w13, bank.w2, bank.w13_scale,
                   bank.w2_scale)

    def c(self) -> moe_experts:
        return moe_experts(DTYPES[self.fmt], self.w13.data_ptr(),
                           self.w13_scale.data_ptr() if self.w13_scale is not None else None,
                           self.w2.data_ptr(),
                           self.w2_scale.data_ptr() if self.w2_scale is not None else None,
                           self.E, self.H, self.I)


def moe_route(x, w_router, bias, k: int, score: str, route_scale: float, topk_idx, topk_w,
              logits=None, ws=None, stream=None):
    T, H = x.shape
    E = w_router.shape[0]
    if ws is None:
        ws = workspace(lib().moe_route_workspace_size(T, H, E), x.device)
    st = lib().moe_route(_ptr(x), _act_dt(x), _ptr(w_router), _ptr(bias), T, H, E, k, SCORES[score],
                         float(route_scale), _ptr(topk_idx), _ptr(topk_w), _ptr(logits), _ptr(ws),
                         ws.numel(), _stream(stream))
    _check(st, "moe_route")


def moe_permute(topk_idx, E: int, counts, offsets, perm_src, inv_perm, x=None, x_perm=None, ws=None,
                stream=None):
    T, k = topk_idx.shape
    H = x.shape[1] if x is not None else 0
    if ws is None:
        ws = workspace(lib().moe_permute_workspace_size(T, k, E), topk_idx.device)
    st = lib().moe_permute(_ptr(topk_idx), T, k, E, _ptr(x), _act_dt(x) if x is not None else 0, H,
                           _ptr(counts), _ptr(offsets), _ptr(perm_src), _ptr(inv_perm), _ptr(x_perm),
                           _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "moe_permute")


def moe_grouped_ffn(experts: Experts, x_perm, offsets, y_perm, ws=None, stream=None):
    rows = x_perm.shape[0]
    cw = experts.c()
    act = _act_dt(x_perm)
    if ws is None:
        ws = workspace(lib().moe_grouped_ffn_workspace_size(ctypes.byref(cw), act, rows), x_perm.device)
    st = lib().moe_grouped_ffn(ctypes.byref(cw), _ptr(x_perm), act, _ptr(offsets), rows, _ptr(y_perm),
                               _act_dt(y_perm), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "moe_grouped_ffn")


def moe_grouped_ffn_prequant(experts: Experts, x_codes, x_scales, offsets, y_perm, ws=None,
                             stream=None):
    """moe_grouped_ffn on rows given as the codes and block scales of moe_quantize_fp8,
    moe_quantize_int8 or moe_quantize_mxfp4 (FP8_E4M3, INT8 and MXFP4_A4 banks)."""
    rows = x_codes.shape[0]
    cw = experts.c()
    if ws is None:
        ws = workspace(lib().moe_grouped_ffn_workspace_size(ctypes.byref(cw), DTYPES["bf16"], rows),
                       x_codes.device)
    st = lib().moe_grouped_ffn_prequant(ctypes.byref(cw), _ptr(x_codes), _ptr(x_scales), _ptr(offsets),
                                        rows, _ptr(y_perm), _act_dt(y_perm), _ptr(ws), ws.numel(),
                                        _stream(stream))
    _check(st, "moe_grouped_ffn_prequant")


def moe_combine(y_perm, inv_perm, topk_w, out, shared_out=None, stream=None):
    T, k = topk_w.shape
    H = out.shape[1]
    st = lib().moe_combine(_ptr(y_perm), _act_dt(y_perm), _ptr(inv_perm), _ptr(topk_w), T, k, H,
                           _ptr(shared_out), _ptr(out), _act_dt(out), _stream(stream))
    _check(st, "moe_combine")


def layer_desc(T: int, wr, bias, routed: Experts, shared: Optional[Experts], k: int, score: str,
               route_scale: float, act_dtype, out_dtype) -> moe_layer_desc:
    d = moe_layer_desc()
    d.T, d.H, d.E, d.k = T, routed.H, routed.E, k
    d.score_fn = SCORES[score]
    d.route_scale = route_scale
    d.act_dtype = act_dtype
    d.out_dtype = out_dtype
    d.w_router = wr.data_ptr()
    d.bias = bias.data_ptr() if bias is not None else None
    d.routed = routed.c()
    d.shared = shared.c() if shared is not None else moe_experts()
    return d


def moe_layer_workspace_size(desc: moe_layer_desc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_layer_workspace_size(ctypes.byref(desc), ctypes.byref(n)), "moe_layer_workspace_size")
    return n.value


def moe_layer_forward(desc: moe_layer_desc, x, out, ws, topk_idx=None, topk_w=None, counts=None,
                      logits=None, stream=None):
    st = lib().moe_layer_forward(ctypes.byref(desc), _ptr(x), _ptr(out), _ptr(topk_idx), _ptr(topk_w),
                                 _ptr(counts), _ptr(logits), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "moe_layer_forward")


NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES of moe.h


def moe_layer_forward_noalloc(desc: moe_layer_desc, x, out, topk_idx=None, topk_w=None,
                              counts=None, logits=None, stream=None):
    """moe_layer_forward on the library's static per-GPU workspace (no workspace argument)."""
    st = lib().moe_layer_forward_noalloc(ctypes.byref(desc), _ptr(x), _ptr(out), _ptr(topk_idx),
                                         _ptr(topk_w), _ptr(counts), _ptr(logits), _stream(stream))
    _check(st, "moe_layer_forward_noalloc")


STAGE_EVENTS = 6
STAGES = ["route", "permute", "gate_up", "down", "combine"]


class StageEvents:
    """MOE_STAGE_EVENTS hipEvent_t handles from the HIP runtime torch has loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = (ctypes.c_void_p * STAGE_EVENTS)()
        for i in range(STAGE_EVENTS):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev[i] = h

    def elapsed_ms(self):
        """Per-stage milliseconds of the last timed call (the stream must be synchronised)."""
        out = []
        for i in range(STAGE_EVENTS - 1):
            ms = ctypes.c_float()
            if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.ev[i], self.ev[i + 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out.append(ms.value)
        return dict(zip(STAGES, out))

    def __del__(self):
        try:
            for i in range(STAGE_EVENTS):
                self.hip.hipEventDestroy(self.ev[i])
        except Exception:
            pass


def moe_layer_forward_timed(desc: moe_layer_desc, x, out, ws, events: StageEvents, topk_idx=None,
                            topk_w=None, counts=None, logits=None, stream=None):
    st = lib().moe_layer_forward_timed(ctypes.byref(desc), _ptr(x), _ptr(out), _ptr(topk_idx),
                                       _ptr(topk_w), _ptr(counts), _ptr(logits), _ptr(ws), ws.numel(),
                                       _stream(stream), events.ev)
    _check(st, "moe_layer_forward_timed")


class ForkJoin:
    """A side stream and the fork/join event pair moe_layer_forward_overlap takes."""

    def __init__(self, device=None):
        self.side = torch.cuda.Stream(device=device)
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(2):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreateWithFlags(ctypes.byref(h), 0x2) != 0:  # timing disabled
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.ev.append(h)

    def __del__(self):
        try:
            for h in self.ev:
                self.hip.hipEventDestroy(h)
        except Exception:
            pass


def moe_layer_forward_overlap(desc: moe_layer_desc, x, out, ws, fj: ForkJoin, topk_idx=None,
                              topk_w=None, counts=None, logits=None, stream=None):
    st = lib().moe_layer_forward_overlap(ctypes.byref(desc), _ptr(x), _ptr(out), _ptr(topk_idx),
                                         _ptr(topk_w), _ptr(counts), _ptr(logits), _ptr(ws),
                                         ws.numel(), _stream(stream), _stream(fj.side), fj.ev[0],
                                         fj.ev[1])
    _check(st, "moe_layer_forward_overlap")


class SplitStreams:
    """Two HIP streams and a fork/join event pair for moe_layer_forward_split. With CU masks
    (lists of 32-bit words, bit i = compute unit i) the streams are created with
    hipExtStreamCreateWithCUMask, so the hot and cold groups run on disjoint compute units;
    without, they share all of them. Both streams keep the default priority."""

    def __init__(self, hot_mask=None, cold_mask=None):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        vpp = ctypes.POINTER(ctypes.c_void_p)
        self.hip.hipStreamCreate.argtypes = [vpp]
        self.hip.hipExtStreamCreateWithCUMask.argtypes = [vpp, ctypes.c_uint32,
                                                          ctypes.POINTER(ctypes.c_uint32)]
        self.hip.hipStreamDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventCreateWithFlags.argtypes = [vpp, ctypes.c_uint]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.streams, self.ev = [], []
        for mask in (hot_mask, cold_mask):
            h = ctypes.c_void_p()
            if mask is None:
                rc = self.hip.hipStreamCreate(ctypes.byref(h))
            else:
                words = (ctypes.c_uint32 * len(mask))(*mask)
                rc = self.hip.hipExtStreamCreateWithCUMask(ctypes.byref(h), len(mask), words)
            if rc != 0:
                raise RuntimeError(f"stream creation failed ({rc})")
            self.streams.append(h)
        for _ in range(2):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreateWithFlags(ctypes.byref(h), 0x2) != 0:  # timing disabled
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.ev.append(h)
        self.hot, self.cold = self.streams

    def __del__(self):
        try:
            for h in self.ev:
                self.hip.hipEventDestroy(h)
            for h in self.streams:
                self.hip.hipStreamDestroy(h)
        except Exception:
            pass


def cu_masks(n_cu: int, cold_share: int = 4):
    """Disjoint CU masks: every cold_share-th group of 8 consecutive CUs for the cold stream,
    the rest for the hot one (whichever way CU numbers map to XCDs -- interleaved or in
    blocks of 32 -- each XCD gets the same split)."""
    hot = [0] * ((n_cu + 31) // 32)
    cold = list(hot)
    for i in range(n_cu):
        m = cold if (i // 8) % cold_share == cold_share - 1 else hot
        m[i // 32] |= 1 << (i % 32)
    return hot, cold


def moe_layer_forward_split(desc: moe_layer_desc, x, out, ws, ss: SplitStreams, cold_rows_max: int,
                            topk_idx=None, topk_w=None, counts=None, logits=None):
    """The layer on ss.hot (route, permute, hot groups, combine) and ss.cold (groups of at most
    cold_rows_max rows). The caller orders ss.hot after the producers of x and before the
    consumers of out (e.g. by synchronising)."""
    st = lib().moe_layer_forward_split(ctypes.byref(desc), _ptr(x), _ptr(out), _ptr(topk_idx),
                                       _ptr(topk_w), _ptr(counts), _ptr(logits), _ptr(ws),
                                       ws.numel(), ss.hot, ss.cold, ss.ev[0], ss.ev[1],
                                       int(cold_rows_max))
    _check(st, "moe_layer_forward_split")


def moe_quantize_fp8(x, q, q_scale, stream=None):
    n, H = x.shape
    st = lib().moe_quantize_fp8(_ptr(x), n, H, _ptr(q), _ptr(q_scale), _stream(stream))
    _check(st, "moe_quantize_fp8")


def moe_quantize_int8(x, q, q_scale, stream=None):
    n, H = x.shape
    st = lib().moe_quantize_int8(_ptr(x), n, H, _ptr(q), _ptr(q_scale), _stream(stream))
    _check(st, "moe_quantize_int8")


def moe_quantize_mxfp4(x, q, q_scale, stream=None):
    n, H = x.shape
    st = lib().moe_quantize_mxfp4(_ptr(x), n, H, _ptr(q), _ptr(q_scale), _stream(stream))
    _check(st, "moe_quantize_mxfp4")


def moe_bias_update(counts, u: float, bias, stream=None):
    """In-place selection-bias step from per-expert routed counts (int32 [E], f32 [E])."""
    if counts.numel() != bias.numel():
        raise ValueError(f"counts has {counts.numel()} experts, bias {bias.numel()}")
    st = lib().moe_bias_update(_ptr(counts), counts.numel(), float(u), _ptr(bias), _stream(stream))
    _check(st, "moe_bias_update")


def moe_probe_hbm_read(buf, sink, stream=None):
    """Measurement probe: one non-temporal streaming read of the whole of `buf` (a device
    tensor of a multiple of 16 bytes); sink: a device int32/uint32 tensor of >= 1 element."""
    st = lib().moe_probe_hbm_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                  _stream(stream))
    _check(st, "moe_probe_hbm_read")


def moe_probe_mfma(dtype: str, iters: int, sink, stream=None) -> float:
    """Measurement probe: `iters` rounds of dense MFMAs ("bf16", "fp8", "int8" or "mxfp4a4",
    the FP4 product) on every CU; returns the operations the launch executes."""
    flops = ctypes.c_double(0.0)
    st = lib().moe_probe_mfma(DTYPES[dtype], int(iters), _ptr(sink), ctypes.byref(flops),
                              _stream(stream))
    _check(st, "moe_probe_mfma")
    return flops.value


def moe_rows_workspace_size(experts: Experts, act_dtype, rows: int) -> int:
    cw = experts.c()
    return lib().moe_rows_workspace_size(ctypes.byref(cw), act_dtype, rows)


def moe_rows_forward(experts: Experts, x, row_expert, row_w, out, ws, stream=None):
    cw = experts.c()
    rows = x.shape[0]
    st = lib().moe_rows_forward(ctypes.byref(cw), _ptr(x), _act_dt(x), _ptr(row_expert), _ptr(row_w),
                                rows, _ptr(out), _act_dt(out), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "moe_rows_forward")


def moe_rows_forward_timed(experts: Experts, x, row_expert, row_w, out, ws, events: StageEvents,
                           stream=None):
    cw = experts.c()
    rows = x.shape[0]
    st = lib().moe_rows_forward_timed(ctypes.byref(cw), _ptr(x), _act_dt(x), _ptr(row_expert),
                                      _ptr(row_w), rows, _ptr(out), _act_dt(out), _ptr(ws),
                                      ws.numel(), _stream(stream), events.ev)
    _check(st, "moe_rows_forward_timed")


class MoELayer:
    """Holds a layer's device weights, its descriptor and a workspace sized once."""

    def __init__(self, T: int, wr, bias, routed: Experts, shared: Optional[Experts], k: int,
                 score: str, route_scale: float, act: str, out: str, device="cuda"):
        self.T, self.k = T, k
        self.wr, self.bias, self.routed, self.shared = wr, bias, routed, shared
        self.act, self.out = act, out
        self.desc = layer_desc(T, wr, bias, routed, shared, k, score, route_scale, DTYPES[act],
                               DTYPES[out])
        self.ws = workspace(moe_layer_workspace_size(self.desc), device)

    @classmethod
    def from_problem(cls, cfg, dev, device="cuda") -> "MoELayer":
        """From a workload description (T, k, score, scale, act, out) and its device tensors
        (wr, bias, routed and shared banks), e.g. those of the seeded workload generator."""
        shared = Experts.from_bank(dev.shared) if dev.shared is not None else None
        return cls(cfg.T, dev.wr, dev.bias, Experts.from_bank(dev.routed), shared, cfg.k,
                   cfg.score, cfg.scale, cfg.act, cfg.out, device)

    def forward(self, x, out, topk_idx=None, topk_w=None, counts=None, logits=None, stream=None):
        moe_layer_forward(self.desc, x, out, self.ws, topk_idx, topk_w, counts, logits, stream)
        return out

    def forward_overlap(self, x, out, fj: ForkJoin, topk_idx=None, topk_w=None, counts=None,
                        logits=None, stream=None):
        moe_layer_forward_overlap(self.desc, x, out, self.ws, fj, topk_idx, topk_w, counts, logits,
                                  stream)
        return out
