"""Seeded synthetic inputs for the MoE layer, on the host and on the device.

Every tensor is a pure function of (seed, tensor id, element index) through the
counter-based Philox4x32-10 generator (Salmon et al., SC 2011), so the host (C)
and device (HIP) fills produce identical bytes, and any slice of a large weight
bank (one expert, say) can be regenerated on the host without the rest.

This module holds no arithmetic of the MoE layer: it makes inputs only, in the
storage formats the layer consumes (fp32, bf16 bits, E4M3FN codes with fp32
128x128 block scales, MXFP4 packed nibbles with e8m0 block scales). Both the
oracle side (tests, the CPU baseline) and the device side use it.
"""
from __future__ import annotations

import ctypes
import os
from functools import lru_cache

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libsynth_host.so")
DEV_LIB = os.path.join(_HERE, "libsynth_dev.so")

QBITS = 16
QN = 1 << QBITS

# tensor ids (third Philox counter word)
TID_X = 1
TID_WR = 2
TID_BIAS = 3
TID_W13 = 4
TID_W2 = 5
TID_WS13 = 6
TID_WS2 = 7
TID_ROWW = 8

_NTHREADS = max(1, min(16, os.cpu_count() or 1))


def build(verbose: bool = False) -> None:
    """Compile the host generator with gcc and the device generator with hipcc."""
    import subprocess

    src = os.path.join(_HERE, "csrc")
    cmds = [
        ["gcc", "-O2", "-fPIC", "-shared", "-std=c99", "-ffp-contract=off", "-pthread",
         os.path.join(src, "synth_host.c"), "-o", HOST_LIB],
        ["hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
         "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         os.path.join(src, "synth_dev.hip"), "-o", DEV_LIB],
    ]
    for c in cmds:
        r = subprocess.run(c, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("synth build failed: " + " ".join(c) + "\n" + r.stdout + r.stderr)
        if verbose:
            print(" ".join(c))


@lru_cache(maxsize=1)
def quantile_table() -> np.ndarray:
    """QN+1 standard-normal quantiles at p_i = (i + 1/2) / (QN + 1), as fp32."""
    from scipy.special import ndtri

    p = (np.arange(QN + 1, dtype=np.float64) + 0.5) / (QN + 1)
    return np.ascontiguousarray(ndtri(p).astype(np.float32))


@lru_cache(maxsize=1)
def _host():
    if not os.path.exists(HOST_LIB):
        build()
    lib = ctypes.CDLL(HOST_LIB)
    u64, u32, i64, f32, vp, ci = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64,
                                  ctypes.c_float, ctypes.c_void_p, ctypes.c_int)
    lib.synth_host_words.argtypes = [u64, u32, u64, u64, vp, ci]
    lib.synth_host_normal_f32.argtypes = [u64, u32, u64, u64, f32, vp, vp, ci]
    lib.synth_host_normal_bf16.argtypes = [u64, u32, u64, u64, f32, vp, vp, ci]
    lib.synth_host_uniform_f32.argtypes = [u64, u32, u64, u64, f32, f32, vp, ci]
    lib.synth_host_fp8_bank.argtypes = [u64, u32, i64, i64, i64, i64, f32, vp, vp, vp, ci]
    lib.synth_host_mxfp4_bank.argtypes = [u64, u32, i64, i64, i64, i64, f32, vp, vp, vp, ci]
    lib.synth_host_int8_bank.argtypes = [u64, u32, i64, i64, i64, i64, f32, vp, vp, vp, ci]
    lib.synth_host_philox_block.argtypes = [vp, vp, vp]
    for f in (lib.synth_host_words, lib.synth_host_normal_f32, lib.synth_host_normal_bf16,
              lib.synth_host_uniform_f32, lib.synth_host_fp8_bank, lib.synth_host_mxfp4_bank,
              lib.synth_host_int8_bank,
              lib.synth_host_philox_block):
        f.restype = None
    return lib


def _p(a: np.ndarray) -> int:
    return a.ctypes.data


# ----------------------------------------------------------------------------- host fills

def philox_block(ctr, key) -> np.ndarray:
    """One Philox4x32-10 output block for counter ctr[4] and key key[2]."""
    c = np.asarray(ctr, np.uint32)
    k = np.asarray(key, np.uint32)
    out = np.empty(4, np.uint32)
    _host().synth_host_philox_block(_p(c), _p(k), _p(out))
    return out


def words(seed: int, tid: int, start: int, n: int) -> np.ndarray:
    out = np.empty(n, np.uint32)
    _host().synth_host_words(seed, tid, start, n, _p(out), _NTHREADS)
    return out


def normal_f32(seed: int, tid: int, shape, std: float, start: int = 0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    q = quantile_table()
    _host().synth_host_normal_f32(seed, tid, start, n, np.float32(std), _p(q), _p(out), _NTHREADS)
    return out.reshape(shape)


def normal_bf16(seed: int, tid: int, shape, std: float, start: int = 0) -> np.ndarray:
    """bf16 bit patterns (uint16) of RNE-rounded N(0, std^2) fp32 values."""
    n = int(np.prod(shape))
    out = np.empty(n, np.uint16)
    q = quantile_table()
    _host().synth_host_normal_bf16(seed, tid, start, n, np.float32(std), _p(q), _p(out), _NTHREADS)
    return out.reshape(shape)


def uniform_f32(seed: int, tid: int, shape, lo: float, hi: float, start: int = 0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    span = np.float32(np.float32(hi) - np.float32(lo))
    _host().synth_host_uniform_f32(seed, tid, start, n, np.float32(lo), span, _p(out), _NTHREADS)
    return out.reshape(shape)


def fp8_bank(seed: int, tid: int, e0: int, ne: int, rows: int, cols: int, std: float):
    """Experts [e0, e0+ne): (codes uint8 [ne,rows,cols], scales f32 [ne,rows/128,cols/128])."""
    codes = np.empty((ne, rows, cols), np.uint8)
    scales = np.empty((ne, rows // 128, cols // 128), np.float32)
    q = quantile_table()
    _host().synth_host_fp8_bank(seed, tid, e0, ne, rows, cols, np.float32(std), _p(q), _p(codes),
                                _p(scales), _NTHREADS)
    return codes, scales


def int8_bank(seed: int, tid: int, e0: int, ne: int, rows: int, cols: int, std: float):
    """Experts [e0, e0+ne): (codes int8 [ne,rows,cols], scales f32 [ne,rows/128,cols/128])."""
    codes = np.empty((ne, rows, cols), np.int8)
    scales = np.empty((ne, rows // 128, cols // 128), np.float32)
    q = quantile_table()
    _host().synth_host_int8_bank(seed, tid, e0, ne, rows, cols, np.float32(std), _p(q), _p(codes),
                                 _p(scales), _NTHREADS)
    return codes, scales


def mxfp4_bank(seed: int, tid: int, e0: int, ne: int, rows: int, cols: int, std: float):
    """Experts [e0, e0+ne): (packed uint8 [ne,rows,cols/2], e8m0 codes uint8 [ne,rows,cols/32])."""
    packed = np.empty((ne, rows, cols // 2), np.uint8)
    scales = np.empty((ne, rows, cols // 32), np.uint8)
    q = quantile_table()
    _host().synth_host_mxfp4_bank(seed, tid, e0, ne, rows, cols, np.float32(std), _p(q),
                                  _p(packed), _p(scales), _NTHREADS)
    return packed, scales


# ----------------------------------------------------------------------------- device fills

@lru_cache(maxsize=1)
def _dev():
    import torch  # noqa: F401  (loads the HIP runtime torch uses before ours binds to it)

    if not os.path.exists(DEV_LIB):
        raise RuntimeError(f"{DEV_LIB} is not built; run synth.build()")
    lib = ctypes.CDLL(DEV_LIB)
    u64, u32, i64, f32, vp = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64, ctypes.c_float,
                              ctypes.c_void_p)
    lib.synth_dev_words.argtypes = [u64, u32, u64, u64, vp, vp]
    lib.synth_dev_normal_bf16.argtypes = [u64, u32, u64, f32, vp, vp, vp]
    lib.synth_dev_normal_f32.argtypes = [u64, u32, u64, f32, vp, vp, vp]
    lib.synth_dev_fp8_bank.argtypes = [u64, u32, i64, i64, i64, i64, f32, vp, vp, vp, vp]
    lib.synth_dev_mxfp4_bank.argtypes = [u64, u32, i64, i64, i64, i64, f32, vp, vp, vp, vp]
    lib.synth_dev_int8_bank.argtypes = [u64, u32, i64, i64, i64, i64, f32, vp, vp, vp, vp]
    for f in (lib.synth_dev_words, lib.synth_dev_normal_bf16, lib.synth_dev_normal_f32,
              lib.synth_dev_fp8_bank, lib.synth_dev_mxfp4_bank, lib.synth_dev_int8_bank):
        f.restype = ctypes.c_int
    return lib


@lru_cache(maxsize=4)
def _dev_table(device: str):
    import torch

    return torch.from_numpy(quantile_table()).to(device)


def _stream():
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _chk(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"synth device fill {what} failed with code {rc}")


def dev_words(seed: int, tid: int, start: int, n: int, device="cuda"):
    import torch

    out = torch.empty(n, dtype=torch.int32, device=device)
    _chk(_dev().synth_dev_words(seed, tid, start, n, out.data_ptr(), _stream()), "words")
    return out


def dev_normal(seed: int, tid: int, shape, std: float, dtype: str, device="cuda"):
    """Device tensor of N(0, std^2): dtype 'bf16' (torch.bfloat16) or 'f32'."""
    import torch

    n = int(np.prod(shape))
    q = _dev_table(str(device))
    if dtype == "bf16":
        out = torch.empty(tuple(shape), dtype=torch.bfloat16, device=device)
        _chk(_dev().synth_dev_normal_bf16(seed, tid, n, np.float32(std), q.data_ptr(),
                                          out.data_ptr(), _stream()), "normal_bf16")
    elif dtype == "f32":
        out = torch.empty(tuple(shape), dtype=torch.float32, device=device)
        _chk(_dev().synth_dev_normal_f32(seed, tid, n, np.float32(std), q.data_ptr(),
                                         out.data_ptr(), _stream()), "normal_f32")
    else:
        raise ValueError(dtype)
    return out


def dev_fp8_bank(seed: int, tid: int, ne: int, rows: int, cols: int, std: float, device="cuda"):
    import torch

    codes = torch.empty((ne, rows, cols), dtype=torch.uint8, device=device)
    scales = torch.empty((ne, rows // 128, cols // 128), dtype=torch.float32, device=device)
    q = _dev_table(str(device))
    _chk(_dev().synth_dev_fp8_bank(seed, tid, 0, ne, rows, cols, np.float32(std), q.data_ptr(),
                                   codes.data_ptr(), scales.data_ptr(), _stream()), "fp8_bank")
    return codes, scales


def dev_int8_bank(seed: int, tid: int, ne: int, rows: int, cols: int, std: float, device="cuda"):
    import torch

    codes = torch.empty((ne, rows, cols), dtype=torch.int8, device=device)
    scales = torch.empty((ne, rows // 128, cols // 128), dtype=torch.float32, device=device)
    q = _dev_table(str(device))
    _chk(_dev().synth_dev_int8_bank(seed, tid, 0, ne, rows, cols, np.float32(std), q.data_ptr(),
                                    codes.data_ptr(), scales.data_ptr(), _stream()), "int8_bank")
    return codes, scales


def dev_mxfp4_bank(seed: int, tid: int, ne: int, rows: int, cols: int, std: float, device="cuda"):
    import torch

    packed = torch.empty((ne, rows, cols // 2), dtype=torch.uint8, device=device)
    scales = torch.empty((ne, rows, cols // 32), dtype=torch.uint8, device=device)
    q = _dev_table(str(device))
    _chk(_dev().synth_dev_mxfp4_bank(seed, tid, 0, ne, rows, cols, np.float32(std), q.data_ptr(),
                                     packed.data_ptr(), scales.data_ptr(), _stream()), "mxfp4_bank")
    return packed, scales
