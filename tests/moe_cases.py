"""Shared helpers of the GPU tests: run the HIP library on a problem and fetch results.

Inputs come from the seeded generator (synth), identical bytes on host and device.
Expected values come only from the oracle, computed on the host from the same bytes.
"""
import os

import numpy as np
import torch

import mixture_experts_layer_04_amd as moe
from synth.configs import MoEConfig
from synth.problem import DevProblem, device_problem, host_problem

# the stated tolerances; INT8 (W8A8) takes the low-precision one of fp8 / MXFP4
TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2, "mxfp4": 6e-2, "mxfp4a4": 6e-2, "int8": 6e-2}

# rows per tile of the grouped FFN kernels the library picks at each full-size workload
TILE_ROWS = {"r1_decode": 16, "r1_decode_fp8": 128, "r1_decode_mxfp4": 16, "r1_prefill": 256,
             "e384_fp8": 128, "ep32_mxfp4": 128, "ep32_w4a4": 128, "r1_decode_int8": 128,
             "r1_prefill_int8": 128}


def experts(bank) -> moe.Experts:
    return moe.Experts.from_bank(bank)


def make_layer(cfg: MoEConfig, dev: DevProblem) -> moe.MoELayer:
    return moe.MoELayer.from_problem(cfg, dev)


def run_layer(cfg: MoEConfig, dev: DevProblem, layer=None, with_logits=True):
    layer = layer or make_layer(cfg, dev)
    T, k, E, H = cfg.T, cfg.k, cfg.E, cfg.H
    dt = torch.float32 if cfg.out == "f32" else torch.bfloat16
    out = torch.empty((T, H), dtype=dt, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda") if with_logits else None
    layer.forward(dev.x, out, idx, w, counts, logits)
    torch.cuda.synchronize()
    res = {"out": out.float().cpu().numpy().astype(np.float64), "topk_idx": idx.cpu().numpy(),
           "topk_w": w.cpu().numpy(), "counts": counts.cpu().numpy()}
    if with_logits:
        res["logits"] = logits.cpu().numpy()
    return res


def run_rows(cfg: MoEConfig, dev: DevProblem):
    rows = cfg.T
    e = experts(dev.routed)
    dt = torch.float32 if cfg.out == "f32" else torch.bfloat16
    out = torch.empty((rows, cfg.H), dtype=dt, device="cuda")
    ws = moe.workspace(moe.moe_rows_workspace_size(e, moe.DTYPES[cfg.act], rows))
    moe.moe_rows_forward(e, dev.x, dev.topk_idx.view(-1), dev.topk_w.view(-1), out, ws)
    torch.cuda.synchronize()
    return {"out": out.float().cpu().numpy().astype(np.float64)}


def problems(cfg: MoEConfig):
    host = host_problem(cfg)
    dev = device_problem(cfg, host=host)
    return host, dev


def describe(cfg: MoEConfig) -> str:
    return (f"{cfg.name}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} I={cfg.I} shared={cfg.shared_I} "
            f"{cfg.score} bias={cfg.use_bias} scale={cfg.scale} {cfg.act}/{cfg.wdt}/{cfg.out}")


def cover_tokens(topk_idx: np.ndarray, E: int, tile_m: int, shared: bool) -> list:
    """Tokens whose outputs together exercise every touched expert and the ragged ends of
    the grouped GEMM tiles: for each expert, the tokens of its first row and of the first
    and last row of its last tile (rows in expert-then-token order, tiles of tile_m rows);
    for the shared group (one row per token), the first and last row of its last tile."""
    import oracle as O

    T, k = topk_idx.shape
    counts, offsets, perm_src, _ = O.permutation(topk_idx, E)
    toks = set()
    for e in range(E):
        c = int(counts[e])
        if c == 0:
            continue
        r0 = int(offsets[e])
        for r in (r0, r0 + (c - 1) // tile_m * tile_m, int(offsets[e + 1]) - 1):
            toks.add(int(perm_src[r]) // k)
    if shared:
        toks.update({(T - 1) // tile_m * tile_m, T - 1})
    return sorted(toks)


class DeviceBytesBank:
    """A host bank whose expert e is read back from the bytes the seeded generator filled in
    HBM (the same bytes as the host generator's: test_device_generator_matches_host), so a
    full-size oracle leg does not generate 20 GB of weights on the CPU again. The tests read
    them before the library's first call on the problem."""

    def __init__(self, host_bank, dev_bank):
        self.fmt, self.E, self.H, self.I = host_bank.fmt, host_bank.E, host_bank.H, host_bank.I
        self._host, self._dev = host_bank, dev_bank

    @staticmethod
    def _np(t):
        t = t.detach().cpu()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    def _part(self, w, sc, e):
        d = {"w": self._np(w[e])}
        if sc is not None:
            d["scale"] = self._np(sc[e])
        return d

    def w13(self, e):
        return self._part(self._dev.w13, self._dev.w13_scale, e)

    def w2(self, e):
        return self._part(self._dev.w2, self._dev.w2_scale, e)

    def spot_check(self, experts):
        """The device bytes of these experts equal the host generator's."""
        for e in experts:
            for a, b in ((self.w13(e), self._host.w13(e)), (self.w2(e), self._host.w2(e))):
                for key in a:
                    assert np.array_equal(a[key], b[key]), (e, key)


def with_device_banks(host, dev):
    """host with its expert banks read from the device fill (first and last expert
    spot-checked against the host generator)."""
    host.routed = DeviceBytesBank(host.routed, dev.routed)
    host.routed.spot_check([0, host.routed.E - 1])
    if host.shared is not None:
        host.shared = DeviceBytesBank(host.shared, dev.shared)
        host.shared.spot_check([0])
    return host


def oracle_layer(host, tokens=None):
    """oracle.layer_forward with the experts evaluated on a pool of threads (each with one
    BLAS thread): the same result as the serial loop, in a fraction of the time."""
    from threadpoolctl import threadpool_limits

    import oracle as O

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with threadpool_limits(1):
        return O.layer_forward(host, tokens=tokens, workers=workers)
