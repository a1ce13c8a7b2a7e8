"""Assemble the inputs of one MoE-layer problem, on the host or on the device.

Host problems hold numpy arrays in storage format (fp32 values, bf16 bit patterns
as uint16, E4M3 codes, packed MXFP4) and generate expert weights lazily, one
expert at a time, so a check of a few tokens of a 22 GB layer only materialises
the experts those tokens use. Device problems hold the same bytes in torch
tensors, generated in HBM by the device fill kernels.

Element numbering (which decides every value): an expert bank of shape [E, R, C]
numbers element (e, r, c) as (e*R + r)*C + c; x [T, H] as t*H + h; the router
[E, H] as e*H + h. fp8 banks are quantised per 128x128 block of each expert's
[R, C] matrix, MXFP4 banks per 32 consecutive elements along C.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import (TID_BIAS, TID_ROWW, TID_W2, TID_W13, TID_WR, TID_WS2, TID_WS13, TID_X,
               fp8_bank, int8_bank, mxfp4_bank, normal_bf16, normal_f32, uniform_f32)
from .configs import MoEConfig


def _bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest even) and return the bit patterns."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


@dataclass
class HostBank:
    """Lazily generated expert bank: W13 [E, 2I, H] (gate rows then up rows), W2 [E, H, I]."""
    fmt: str
    E: int
    H: int
    I: int
    seed: int
    tid13: int
    tid2: int
    std: float

    def _dense(self, tid: int, e: int, rows: int, cols: int):
        start = e * rows * cols
        if self.fmt == "bf16":
            return {"w": normal_bf16(self.seed, tid, (rows, cols), self.std, start=start)}
        if self.fmt == "f32":
            return {"w": normal_f32(self.seed, tid, (rows, cols), self.std, start=start)}
        if self.fmt == "fp8":
            c, s = fp8_bank(self.seed, tid, e, 1, rows, cols, self.std)
            return {"w": c[0], "scale": s[0]}
        if self.fmt == "int8":
            c, s = int8_bank(self.seed, tid, e, 1, rows, cols, self.std)
            return {"w": c[0], "scale": s[0]}
        if self.fmt in ("mxfp4", "mxfp4a4"):
            p, s = mxfp4_bank(self.seed, tid, e, 1, rows, cols, self.std)
            return {"w": p[0], "scale": s[0]}
        raise ValueError(self.fmt)

    def w13(self, e: int) -> dict:
        return self._dense(self.tid13, e, 2 * self.I, self.H)

    def w2(self, e: int) -> dict:
        return self._dense(self.tid2, e, self.H, self.I)


@dataclass
class HostProblem:
    cfg: MoEConfig
    x: np.ndarray                       # [T, H] f32 or bf16 bits
    wr: Optional[np.ndarray]            # [E, H] same storage as x (None: pre-routed rows)
    bias: Optional[np.ndarray]          # [E] f32
    routed: HostBank
    shared: Optional[HostBank]
    topk_idx: Optional[np.ndarray] = None   # pre-routed rows: [T, 1] int32
    topk_w: Optional[np.ndarray] = None     # pre-routed rows: [T, 1] f32


def zipf_offsets(cfg: MoEConfig) -> np.ndarray:
    """Per-expert router-row offset gamma * r_e^(-s), r_e a seeded permutation of 1..E, fp32."""
    rng = np.random.default_rng(cfg.seed + 17)
    ranks = rng.permutation(cfg.E).astype(np.float64) + 1.0
    z = (ranks ** (-cfg.zipf_s)).astype(np.float32)
    return (np.float32(cfg.zipf_gamma) * z).astype(np.float32)


def router_weights(cfg: MoEConfig) -> np.ndarray:
    """Router [E, H] in activation storage; with a Zipf offset, bf16(fp32(w) + offset_e)."""
    if cfg.zipf_s:
        w = normal_f32(cfg.weight_seed, TID_WR, (cfg.E, cfg.H), cfg.w_std)
        w = (w + zipf_offsets(cfg)[:, None]).astype(np.float32)
        if cfg.act == "bf16":
            return _bf16_bits_from_f32(w)
        return w
    if cfg.act == "bf16":
        return normal_bf16(cfg.weight_seed, TID_WR, (cfg.E, cfg.H), cfg.w_std)
    return normal_f32(cfg.weight_seed, TID_WR, (cfg.E, cfg.H), cfg.w_std)


def preroute(cfg: MoEConfig):
    """Pre-routed rows: Dirichlet(alpha) expert shares, multinomial counts over T rows,
    expert ids in a seeded shuffled order, row weights U(0, 1)."""
    rng = np.random.default_rng(cfg.seed + 29)
    p = rng.dirichlet(np.full(cfg.E, cfg.dirichlet_alpha))
    counts = rng.multinomial(cfg.T, p)
    ids = np.repeat(np.arange(cfg.E, dtype=np.int32), counts)
    ids = ids[rng.permutation(cfg.T)]
    w = uniform_f32(cfg.seed, TID_ROWW, (cfg.T,), 0.0, 1.0)
    return ids.reshape(cfg.T, 1).astype(np.int32), w.reshape(cfg.T, 1)


def host_problem(cfg: MoEConfig) -> HostProblem:
    if cfg.act == "bf16":
        x = normal_bf16(cfg.seed, TID_X, (cfg.T, cfg.H), cfg.x_std)
    else:
        x = normal_f32(cfg.seed, TID_X, (cfg.T, cfg.H), cfg.x_std)
    routed = HostBank(cfg.wdt, cfg.E, cfg.H, cfg.I, cfg.weight_seed, TID_W13, TID_W2, cfg.w_std)
    shared = (HostBank(cfg.wdt, 1, cfg.H, cfg.shared_I, cfg.weight_seed, TID_WS13, TID_WS2,
                       cfg.w_std) if cfg.shared_I else None)
    if not cfg.routed:
        idx, w = preroute(cfg)
        return HostProblem(cfg, x, None, None, routed, shared, idx, w)
    wr = router_weights(cfg)
    bias = (uniform_f32(cfg.weight_seed, TID_BIAS, (cfg.E,), cfg.bias_lo, cfg.bias_hi)
            if cfg.use_bias else None)
    return HostProblem(cfg, x, wr, bias, routed, shared)


# ----------------------------------------------------------------------------- device side

@dataclass
class DevBank:
    fmt: str
    E: int
    H: int
    I: int
    w13: object
    w2: object
    w13_scale: object = None
    w2_scale: object = None


@dataclass
class DevProblem:
    cfg: MoEConfig
    x: object
    wr: object
    bias: object
    routed: DevBank
    shared: Optional[DevBank]
    topk_idx: object = None
    topk_w: object = None


def _dev_bank(cfg: MoEConfig, E: int, I: int, tid13: int, tid2: int, device) -> DevBank:
    from . import dev_fp8_bank, dev_int8_bank, dev_mxfp4_bank, dev_normal

    s, H, std = cfg.weight_seed, cfg.H, cfg.w_std
    if cfg.wdt in ("bf16", "f32"):
        return DevBank(cfg.wdt, E, H, I, dev_normal(s, tid13, (E, 2 * I, H), std, cfg.wdt, device),
                       dev_normal(s, tid2, (E, H, I), std, cfg.wdt, device))
    if cfg.wdt in ("fp8", "int8"):
        gen = dev_fp8_bank if cfg.wdt == "fp8" else dev_int8_bank
        c13, s13 = gen(s, tid13, E, 2 * I, H, std, device)
        c2, s2 = gen(s, tid2, E, H, I, std, device)
        return DevBank(cfg.wdt, E, H, I, c13, c2, s13, s2)
    if cfg.wdt in ("mxfp4", "mxfp4a4"):  # the same weights; mxfp4a4 also quantises activations
        p13, s13 = dev_mxfp4_bank(s, tid13, E, 2 * I, H, std, device)
        p2, s2 = dev_mxfp4_bank(s, tid2, E, H, I, std, device)
        return DevBank(cfg.wdt, E, H, I, p13, p2, s13, s2)
    raise ValueError(cfg.wdt)


def _to_dev(a: np.ndarray, device):
    import torch

    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def device_problem(cfg: MoEConfig, device="cuda", host: Optional[HostProblem] = None,
                   banks_of: Optional[DevProblem] = None) -> DevProblem:
    """Inputs in HBM. Large tensors are filled on the device; small ones are uploaded
    from the host generator (same bytes either way). banks_of: a device problem whose
    expert banks are the same bytes (same weight seed, format and shapes), reused instead
    of generated again."""
    from . import dev_normal

    x = dev_normal(cfg.seed, TID_X, (cfg.T, cfg.H), cfg.x_std, cfg.act, device)
    if banks_of is not None:
        o = banks_of.cfg
        same = (o.weight_seed, o.wdt, o.E, o.H, o.I, o.shared_I, o.w_std) == \
               (cfg.weight_seed, cfg.wdt, cfg.E, cfg.H, cfg.I, cfg.shared_I, cfg.w_std)
        if not same:
            raise ValueError(f"{o.name} and {cfg.name} do not share their expert banks")
        routed, shared = banks_of.routed, banks_of.shared
    else:
        routed = _dev_bank(cfg, cfg.E, cfg.I, TID_W13, TID_W2, device)
        shared = _dev_bank(cfg, 1, cfg.shared_I, TID_WS13, TID_WS2, device) if cfg.shared_I else None
    if not cfg.routed:
        idx, w = preroute(cfg) if host is None else (host.topk_idx, host.topk_w)
        return DevProblem(cfg, x, None, None, routed, shared, _to_dev(idx, device),
                          _to_dev(w, device))
    wr = router_weights(cfg) if host is None else host.wr
    bias = None
    if cfg.use_bias:
        bias = (uniform_f32(cfg.weight_seed, TID_BIAS, (cfg.E,), cfg.bias_lo, cfg.bias_hi)
                if host is None else host.bias)
    return DevProblem(cfg, x, _to_dev(wr, device), None if bias is None else _to_dev(bias, device),
                      routed, shared)
