"""Calibrates the router-row Zipf offset amplitude of the r1_prefill workload.

The workload asks for skewed routing in which the top 10% of experts take about
40% of the assignments, produced by an additive per-expert Zipf(s=1.1) offset on
the router weight rows. This script bisects the offset amplitude gamma, routing
all 8192 tokens with the oracle each time, until the 26 most loaded of the 256
experts hold 40% of the 65,536 assignments, and prints gamma. The printed value
is stored as PREFILL_ZIPF_GAMMA in synth/configs.py.

Run: python tests/calibrate_prefill_skew.py
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import oracle as O  # noqa: E402
from synth import TID_BIAS, TID_X, normal_bf16, uniform_f32  # noqa: E402
from synth.configs import CONFIGS  # noqa: E402
from synth.problem import router_weights  # noqa: E402


def top_share(cfg, x64, bias) -> float:
    wr = O.bf16_to_f64(router_weights(cfg))
    r = O.route(x64, wr, bias, cfg.k, cfg.score, cfg.scale)
    counts = np.bincount(r["topk_idx"].reshape(-1), minlength=cfg.E)
    ntop = -(-cfg.E // 10)
    return float(np.sort(counts)[::-1][:ntop].sum() / counts.sum())


def main():
    base = CONFIGS["r1_prefill"]
    x64 = O.bf16_to_f64(normal_bf16(base.seed, TID_X, (base.T, base.H), base.x_std))
    bias = uniform_f32(base.weight_seed, TID_BIAS, (base.E,), base.bias_lo, base.bias_hi)
    lo, hi = 0.0, 0.05
    while top_share(base.with_(zipf_gamma=hi), x64, bias) < 0.40:
        lo, hi = hi, hi * 2
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        sh = top_share(base.with_(zipf_gamma=mid), x64, bias)
        print(f"gamma={mid:.8f} top10%={sh:.4f}", flush=True)
        if abs(sh - 0.40) < 0.0025:
            break
        lo, hi = (mid, hi) if sh < 0.40 else (lo, mid)
    print(f"PREFILL_ZIPF_GAMMA = {mid!r}")


if __name__ == "__main__":
    main()
