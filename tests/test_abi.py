"""The C ABI on the CPU: libmoe.so loads, exports every entry point include/moe.h declares,
its structs have the layout the binding mirrors, and every validation error is returned
before anything is launched (no GPU needed: invalid calls never reach HIP)."""
import ctypes
import os
import re
import subprocess

import pytest

import mixture_experts_layer_04_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

P = 0x10000          # a 256-byte-aligned stand-in for a device pointer (never dereferenced)
MISALIGNED = 0x10008


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:moe_status|size_t|const char\*)\s+(moe_\w+)\(", text, re.M)))


def test_header_functions_are_exported():
    L = moe.lib()
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n
    assert set(names) <= set(moe.EXPORTS)


def test_struct_layout_matches_binding(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "moe.h"\n'
        "int main(void){printf(\"%zu %zu %zu %zu %zu %zu\\n\", sizeof(moe_experts), "
        "sizeof(moe_layer_desc), offsetof(moe_experts, E), offsetof(moe_layer_desc, w_router), "
        "offsetof(moe_layer_desc, routed), offsetof(moe_layer_desc, shared)); return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    want = [ctypes.sizeof(moe.moe_experts), ctypes.sizeof(moe.moe_layer_desc),
            moe.moe_experts.E.offset, moe.moe_layer_desc.w_router.offset,
            moe.moe_layer_desc.routed.offset, moe.moe_layer_desc.shared.offset]
    assert got == want


def test_status_strings():
    L = moe.lib()
    for s in range(7):
        assert L.moe_status_str(s)
    assert L.moe_status_str(99) == b"unknown status"


def route(**kw):
    a = dict(x=P, x_dt=moe.MOE_BF16, wr=P, bias=None, T=4, H=64, E=8, k=2, fn=moe.MOE_SIGMOID,
             scale=1.0, idx=P, w=P, logits=None, ws=P, ws_bytes=1 << 30)
    a.update(kw)
    return moe.lib().moe_route(a["x"], a["x_dt"], a["wr"], a["bias"], a["T"], a["H"], a["E"], a["k"],
                               a["fn"], a["scale"], a["idx"], a["w"], a["logits"], a["ws"],
                               a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=9), moe.MOE_ERR_SHAPE), (dict(k=0), moe.MOE_ERR_SHAPE), (dict(E=1025, k=2), moe.MOE_ERR_SHAPE),
    (dict(E=40, k=17), moe.MOE_ERR_SHAPE), (dict(H=60), moe.MOE_ERR_SHAPE), (dict(T=-1), moe.MOE_ERR_SHAPE),
    (dict(fn=7), moe.MOE_ERR_SHAPE), (dict(x_dt=moe.MOE_FP8_E4M3), moe.MOE_ERR_DTYPE),
    (dict(x=None), moe.MOE_ERR_NULL), (dict(idx=None), moe.MOE_ERR_NULL), (dict(ws=None), moe.MOE_ERR_NULL),
    (dict(x=MISALIGNED), moe.MOE_ERR_ALIGN), (dict(ws=P + 16), moe.MOE_ERR_ALIGN),
    (dict(ws_bytes=16), moe.MOE_ERR_WORKSPACE),
])
def test_route_validation(kw, status):
    assert route(**kw) == status


def test_route_empty_batch_is_ok_without_launch():
    assert route(T=0, x=None, idx=None, w=None, ws=None) == moe.MOE_OK


def test_route_workspace_size():
    L = moe.lib()
    assert L.moe_route_workspace_size(128, 7168, 256) > 0
    assert L.moe_route_workspace_size(-1, 7168, 256) == 0


def bank(fmt="bf16", E=8, H=256, I=128, scales=False):
    return moe.moe_experts(moe.DTYPES[fmt], P, P if scales else None, P, P if scales else None, E, H, I)


def desc(**kw):
    d = moe.moe_layer_desc()
    d.T, d.H, d.E, d.k = kw.get("T", 16), kw.get("H", 256), kw.get("E", 8), kw.get("k", 2)
    d.score_fn = kw.get("score_fn", moe.MOE_SOFTMAX)
    d.route_scale = 1.0
    d.act_dtype = kw.get("act", moe.MOE_BF16)
    d.out_dtype = kw.get("out", moe.MOE_BF16)
    d.w_router = kw.get("wr", P)
    d.bias = kw.get("bias", None)
    d.routed = kw.get("routed", bank(E=d.E, H=d.H))
    d.shared = kw.get("shared", moe.moe_experts())
    return d


def ws_size(d):
    n = ctypes.c_size_t(0)
    return moe.lib().moe_layer_workspace_size(ctypes.byref(d), ctypes.byref(n)), n.value


@pytest.mark.parametrize("kw,status", [
    (dict(k=9), moe.MOE_ERR_SHAPE),
    (dict(E=1024, routed=bank(E=1024), shared=bank(E=1)), moe.MOE_ERR_SHAPE),  # E + shared > 1024
    (dict(routed=bank(E=7)), moe.MOE_ERR_SHAPE),                               # bank E != E
    (dict(routed=bank(H=128)), moe.MOE_ERR_SHAPE),                             # bank H != H
    (dict(H=204, routed=bank(H=204)), moe.MOE_ERR_SHAPE),                      # H % 8
    (dict(routed=bank(I=100)), moe.MOE_ERR_SHAPE),                             # I % 8
    (dict(act=moe.MOE_F32), moe.MOE_ERR_DTYPE),                                # f32 act, bf16 weights
    (dict(out=moe.MOE_FP8_E4M3), moe.MOE_ERR_DTYPE),
    (dict(shared=bank("f32", E=1)), moe.MOE_ERR_DTYPE),                        # shared dtype differs
    (dict(shared=bank(E=2)), moe.MOE_ERR_SHAPE),                               # shared E != 1
    (dict(routed=bank("fp8")), moe.MOE_ERR_NULL),                              # fp8 without scales
    (dict(routed=bank("fp8", H=256, I=192, scales=True)), moe.MOE_ERR_SHAPE),  # fp8 I % 128
    (dict(routed=bank("mxfp4", scales=False)), moe.MOE_ERR_NULL),
    (dict(wr=None), moe.MOE_ERR_NULL),
    (dict(wr=MISALIGNED), moe.MOE_ERR_ALIGN),
    (dict(routed=moe.moe_experts(moe.MOE_BF16, MISALIGNED, None, P, None, 8, 256, 128)), moe.MOE_ERR_ALIGN),
    (dict(score_fn=5), moe.MOE_ERR_SHAPE),
])
def test_layer_validation(kw, status):
    d = desc(**kw)
    st, _ = ws_size(d)
    assert st == status
    assert moe.lib().moe_layer_forward(ctypes.byref(d), P, P, None, None, None, None, P, 1 << 40,
                                       None) == status


@pytest.mark.parametrize("kw", [dict(H=200, routed=bank(H=200)),              # H % 8, not % 64
                                dict(routed=bank(I=136), shared=bank(E=1, I=72)),
                                dict(H=136, act=moe.MOE_F32, out=moe.MOE_F32,
                                     routed=bank("f32", H=136, I=200))])
def test_layer_accepts_multiples_of_8(kw):
    """bf16 and fp32 layers whose H or I is a multiple of 8 but not of 64 are accepted (they
    run on the plain dot-product kernels), and their workspace holds h in fp32."""
    st, n = ws_size(desc(**kw))
    assert st == moe.MOE_OK and n > 0


def test_layer_workspace_and_call_errors():
    d = desc(shared=bank(E=1))
    st, n = ws_size(d)
    assert st == moe.MOE_OK and n > 0
    L = moe.lib()
    assert L.moe_layer_forward(ctypes.byref(d), P, P, None, None, None, None, P, n - 1, None) == \
        moe.MOE_ERR_WORKSPACE
    assert L.moe_layer_forward(ctypes.byref(d), None, P, None, None, None, None, P, n, None) == \
        moe.MOE_ERR_NULL
    assert L.moe_layer_forward(ctypes.byref(d), P, P, MISALIGNED, None, None, None, P, n, None) == \
        moe.MOE_ERR_ALIGN
    assert L.moe_layer_forward(None, P, P, None, None, None, None, P, n, None) == moe.MOE_ERR_NULL
    assert L.moe_layer_forward_timed(ctypes.byref(d), P, P, None, None, None, None, P, n, None,
                                     None) == moe.MOE_ERR_NULL


def test_workspace_grows_with_tokens():
    a, b = ws_size(desc(T=16))[1], ws_size(desc(T=4096))[1]
    assert b > a


def test_other_entry_point_validation():
    L = moe.lib()
    b = bank()
    assert L.moe_permute(P, 4, 9, 8, None, 0, 0, P, P, P, P, None, P, 1 << 30, None) == moe.MOE_ERR_SHAPE
    assert L.moe_permute(P, 4, 2, 8, P, moe.MOE_BF16, 64, P, P, P, P, None, P, 1 << 30, None) == \
        moe.MOE_ERR_NULL                                   # x without x_perm
    assert L.moe_permute(P, 4, 2, 8, None, 0, 0, P, P, P, P, None, P, 0, None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_grouped_ffn(ctypes.byref(b), P, moe.MOE_F32, P, 64, P, moe.MOE_F32, P, 1 << 30,
                             None) == moe.MOE_ERR_DTYPE   # f32 rows with bf16 weights
    assert L.moe_grouped_ffn(ctypes.byref(b), P, moe.MOE_BF16, None, 64, P, moe.MOE_F32, P, 1 << 30,
                             None) == moe.MOE_ERR_NULL
    assert L.moe_grouped_ffn(ctypes.byref(b), P, moe.MOE_BF16, P, 64, P, moe.MOE_F32, P, 16,
                             None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_combine(P, moe.MOE_BF16, P, P, 4, 2, 60, None, P, moe.MOE_BF16, None) == moe.MOE_ERR_SHAPE
    assert L.moe_combine(P, moe.MOE_FP8_E4M3, P, P, 4, 2, 64, None, P, moe.MOE_BF16, None) == \
        moe.MOE_ERR_DTYPE
    assert L.moe_combine(None, moe.MOE_BF16, P, P, 0, 2, 64, None, None, moe.MOE_BF16, None) == moe.MOE_OK
    assert L.moe_quantize_fp8(P, 4, 200, P, P, None) == moe.MOE_ERR_SHAPE
    assert L.moe_quantize_fp8(None, 4, 256, P, P, None) == moe.MOE_ERR_NULL
    assert L.moe_quantize_fp8(P, 0, 256, None, None, None) == moe.MOE_OK
    assert L.moe_rows_forward(ctypes.byref(b), P, moe.MOE_BF16, P, P, 16, P, moe.MOE_BF16, P, 16,
                              None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_rows_forward_timed(ctypes.byref(b), P, moe.MOE_BF16, P, P, 16, P, moe.MOE_BF16, P,
                                    1 << 30, None, None) == moe.MOE_ERR_NULL   # no events
    for H, I in ((192, 128), (256, 192)):                  # MXFP4 needs H % 128 and I % 128
        fb = bank("mxfp4", H=H, I=I, scales=True)
        assert L.moe_rows_forward(ctypes.byref(fb), P, moe.MOE_BF16, P, P, 16, P, moe.MOE_BF16, P,
                                  1 << 30, None) == moe.MOE_ERR_SHAPE


def test_grouped_ffn_prequant_validation():
    """moe_grouped_ffn_prequant takes FP8_E4M3, INT8 and MXFP4_A4 banks only, and checks its
    pointers, alignment and workspace before any launch."""
    L = moe.lib()
    f = L.moe_grouped_ffn_prequant
    for fmt in ("bf16", "mxfp4"):                          # formats without quantised rows
        b = bank(fmt, H=256, I=128, scales=fmt == "mxfp4")
        assert f(ctypes.byref(b), P, P, P, 64, P, moe.MOE_BF16, P, 1 << 30, None) == moe.MOE_ERR_DTYPE
    for fmt in ("fp8", "int8", "mxfp4a4"):
        b = bank(fmt, H=256, I=128, scales=True)
        need = L.moe_grouped_ffn_workspace_size(ctypes.byref(b), moe.MOE_BF16, 64)
        assert need > 0
        assert f(ctypes.byref(b), P, P, P, 64, P, moe.MOE_FP8_E4M3, P, need, None) == moe.MOE_ERR_DTYPE
        assert f(ctypes.byref(b), P, None, P, 64, P, moe.MOE_BF16, P, need, None) == moe.MOE_ERR_NULL
        assert f(ctypes.byref(b), None, P, P, 64, P, moe.MOE_BF16, P, need, None) == moe.MOE_ERR_NULL
        assert f(ctypes.byref(b), P, P, None, 64, P, moe.MOE_BF16, P, need, None) == moe.MOE_ERR_NULL
        assert f(ctypes.byref(b), P, MISALIGNED, P, 64, P, moe.MOE_BF16, P, need, None) == \
            moe.MOE_ERR_ALIGN
        assert f(ctypes.byref(b), P, P, P, 64, P, moe.MOE_BF16, P, need - 1, None) == \
            moe.MOE_ERR_WORKSPACE
        assert f(ctypes.byref(b), P, P, P, -1, P, moe.MOE_BF16, P, need, None) == moe.MOE_ERR_SHAPE
    assert f(None, P, P, P, 64, P, moe.MOE_BF16, P, 1 << 30, None) == moe.MOE_ERR_NULL


def test_bias_update_validation():
    L = moe.lib()
    for E in (0, 1025, -3):
        assert L.moe_bias_update(P, E, 0.01, P, None) == moe.MOE_ERR_SHAPE
    for u in (float("inf"), float("-inf"), float("nan")):
        assert L.moe_bias_update(P, 8, u, P, None) == moe.MOE_ERR_SHAPE
    assert L.moe_bias_update(None, 8, 0.01, P, None) == moe.MOE_ERR_NULL
    assert L.moe_bias_update(P, 8, 0.01, None, None) == moe.MOE_ERR_NULL
    assert L.moe_bias_update(MISALIGNED, 8, 0.01, P, None) == moe.MOE_ERR_ALIGN
    assert L.moe_bias_update(P, 8, 0.01, MISALIGNED, None) == moe.MOE_ERR_ALIGN


def test_layer_overlap_needs_both_events():
    L = moe.lib()
    d = desc(T=16)
    n = ws_size(d)[1]
    for fork, join in ((None, P), (P, None), (None, None)):
        assert L.moe_layer_forward_overlap(ctypes.byref(d), P, P, None, None, None, None, P, n,
                                           None, None, fork, join) == moe.MOE_ERR_NULL
    # the same argument checks as moe_layer_forward come first after the events
    assert L.moe_layer_forward_overlap(ctypes.byref(d), P, P, None, None, None, None, P, 16,
                                       None, None, P, P) == moe.MOE_ERR_WORKSPACE


def test_quantize_mxfp4_validation():
    L = moe.lib()
    assert L.moe_quantize_mxfp4(P, 4, 48, P, P, None) == moe.MOE_ERR_SHAPE
    assert L.moe_quantize_mxfp4(None, 4, 64, P, P, None) == moe.MOE_ERR_NULL
    assert L.moe_quantize_mxfp4(P, 0, 64, None, None, None) == moe.MOE_OK
    assert L.moe_quantize_mxfp4(MISALIGNED, 4, 64, P, P, None) == moe.MOE_ERR_ALIGN
    b = bank("mxfp4a4", H=256, I=192, scales=True)         # I not a multiple of 128
    assert L.moe_rows_forward(ctypes.byref(b), P, moe.MOE_BF16, P, P, 16, P, moe.MOE_BF16, P,
                              1 << 30, None) == moe.MOE_ERR_SHAPE
    b = bank("mxfp4a4", H=256, I=128, scales=True)
    assert L.moe_rows_forward(ctypes.byref(b), P, moe.MOE_F32, P, P, 16, P, moe.MOE_BF16, P,
                              1 << 30, None) == moe.MOE_ERR_DTYPE   # activations must be bf16


def test_noalloc_rejects_layers_beyond_its_static_workspace():
    """moe_layer_forward_noalloc refuses, before any HIP call, a layer whose workspace exceeds
    MOE_NOALLOC_SCRATCH_BYTES (here a 8192-token prefill batch: 2.4 GB)."""
    L = moe.lib()
    d = moe.moe_layer_desc()
    d.T, d.H, d.E, d.k = 8192, 7168, 256, 8
    d.score_fn, d.route_scale = moe.MOE_SIGMOID, 2.5
    d.act_dtype = d.out_dtype = moe.MOE_BF16
    d.w_router = P
    d.routed = moe.moe_experts(moe.MOE_BF16, P, None, P, None, 256, 7168, 2048)
    d.shared = moe.moe_experts(moe.MOE_BF16, P, None, P, None, 1, 7168, 2048)
    n = ctypes.c_size_t(0)
    assert L.moe_layer_workspace_size(ctypes.byref(d), ctypes.byref(n)) == moe.MOE_OK
    assert n.value > moe.NOALLOC_SCRATCH_BYTES
    st = L.moe_layer_forward_noalloc(ctypes.byref(d), P, P, None, None, None, None, None)
    assert st == moe.MOE_ERR_WORKSPACE
    # and the usual argument checks come first
    d.k = 300
    assert L.moe_layer_forward_noalloc(ctypes.byref(d), P, P, None, None, None, None, None) == moe.MOE_ERR_SHAPE


def test_probe_validation():
    """The measurement probes check their arguments before any launch."""
    L = moe.lib()
    f = ctypes.c_double(0.0)
    assert L.moe_probe_hbm_read(P, 0, P, None) == moe.MOE_ERR_SHAPE
    assert L.moe_probe_hbm_read(P, 1000, P, None) == moe.MOE_ERR_SHAPE   # not a multiple of 16
    assert L.moe_probe_hbm_read(None, 1024, P, None) == moe.MOE_ERR_NULL
    assert L.moe_probe_hbm_read(P, 1024, None, None) == moe.MOE_ERR_NULL
    assert L.moe_probe_hbm_read(MISALIGNED, 1024, P, None) == moe.MOE_ERR_ALIGN
    assert L.moe_probe_mfma(moe.MOE_F32, 10, P, ctypes.byref(f), None) == moe.MOE_ERR_DTYPE
    assert L.moe_probe_mfma(moe.MOE_MXFP4, 10, P, ctypes.byref(f), None) == moe.MOE_ERR_DTYPE
    assert L.moe_probe_mfma(moe.MOE_BF16, 0, P, ctypes.byref(f), None) == moe.MOE_ERR_SHAPE
    assert L.moe_probe_mfma(moe.MOE_BF16, 10, None, ctypes.byref(f), None) == moe.MOE_ERR_NULL
    assert L.moe_probe_mfma(moe.MOE_BF16, 10, P, None, None) == moe.MOE_ERR_NULL
