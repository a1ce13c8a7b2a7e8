"""The MoE-layer workloads: shapes, formats and input distributions.

The five named workloads are the ones the layer is measured and checked on:
  tiny_fp32      T=64 H=128 E=8 top-2 I=256, softmax router, fp32, no bias, no shared expert
  r1_decode      T=128 H=7168 E=256 top-8 I=2048, sigmoid + selection bias U(-0.1,0.1),
                 weights renormalised and scaled by 2.5, one shared expert (I=2048), bf16
  r1_prefill     r1_decode at T=8192 with a Zipf(1.1) per-expert offset on the router rows
                 so that the top 10% of experts take about 40% of the assignments
  e384_fp8       T=4096 H=7168 E=384 top-8 I=2048, softmax, one shared expert; E4M3 weights
                 with fp32 128x128 block scales, activations quantised to E4M3 per 1x128
                 with fp32 scales, bf16 output
  ep32_mxfp4     one GPU's expert-parallel share: 32 local experts, 16384 received rows
                 with Dirichlet(0.5)-multinomial expert counts, MXFP4 weights, bf16 rows
The DeepSeek-R1 shape (256 routed + 1 shared expert, 8 distinct experts per token) and
the 384-expert top-8 + shared layout are the ones the MoE pages describe (the WideEP
claim card's context paragraph; the Baidu MoE explainer's "Routing: Top-K Experts Plus
a Shared Expert" section).

All inputs are N(0,1) activations and N(0, 0.02^2) weights from the seeded generator.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int                      # tokens (ep32_mxfp4: received rows)
    H: int                      # hidden size
    E: int                      # routed experts
    k: int                      # experts per token
    I: int                      # routed expert intermediate size
    score: str = "softmax"      # 'softmax' | 'sigmoid' | 'none' (rows arrive pre-routed)
    use_bias: bool = False      # selection-only per-expert bias U(-0.1, 0.1)
    scale: float = 1.0          # routed-weight scale after renormalisation
    shared_I: int = 0           # shared-expert intermediate size (0: no shared expert)
    act: str = "bf16"           # activation storage: 'f32' | 'bf16'
    wdt: str = "bf16"           # expert weight storage: 'f32' | 'bf16' | 'fp8' | 'int8' | 'mxfp4'
    out: str = "bf16"           # output storage: 'f32' | 'bf16'
    seed: int = 0               # seed of x (and of everything else unless weight_seed is set)
    weight_seed: int = 0        # seed of router / expert / shared weights
    zipf_s: float = 0.0         # router-row Zipf offset exponent (0: none)
    zipf_gamma: float = 0.0     # its amplitude
    dirichlet_alpha: float = 0.0  # pre-routed rows: Dirichlet concentration of expert loads
    w_std: float = 0.02
    x_std: float = 1.0
    bias_lo: float = -0.1
    bias_hi: float = 0.1
    tags: tuple = field(default_factory=tuple)

    @property
    def routed(self) -> bool:
        return self.score != "none"

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


# Router-row offset amplitude for r1_prefill, calibrated by
# tests/calibrate_prefill_skew.py with the oracle's routing so that the 26 most
# loaded of 256 experts (the top 10%) take 40% +- 1% of the 65,536 assignments.
PREFILL_ZIPF_GAMMA = 0.2125

CONFIGS = {
    "tiny_fp32": MoEConfig("tiny_fp32", T=64, H=128, E=8, k=2, I=256, score="softmax",
                           act="f32", wdt="f32", out="f32", seed=1000, weight_seed=1000),
    "r1_decode": MoEConfig("r1_decode", T=128, H=7168, E=256, k=8, I=2048, score="sigmoid",
                           use_bias=True, scale=2.5, shared_I=2048, seed=2000, weight_seed=2000),
    "r1_prefill": MoEConfig("r1_prefill", T=8192, H=7168, E=256, k=8, I=2048, score="sigmoid",
                            use_bias=True, scale=2.5, shared_I=2048, seed=3000, weight_seed=2000,
                            zipf_s=1.1, zipf_gamma=PREFILL_ZIPF_GAMMA),
    "e384_fp8": MoEConfig("e384_fp8", T=4096, H=7168, E=384, k=8, I=2048, score="softmax",
                          shared_I=2048, act="bf16", wdt="fp8", out="bf16", seed=4000,
                          weight_seed=4000),
    "ep32_mxfp4": MoEConfig("ep32_mxfp4", T=16384, H=7168, E=32, k=1, I=2048, score="none",
                            act="bf16", wdt="mxfp4", out="bf16", seed=5000, weight_seed=5000,
                            dirichlet_alpha=0.5),
    # r1_decode with the expert weights in fp8 or MXFP4, the low-precision grouped GEMM
    # formats of the GC-MoE record: same seeds, so the same router and routing
    "r1_decode_fp8": MoEConfig("r1_decode_fp8", T=128, H=7168, E=256, k=8, I=2048,
                               score="sigmoid", use_bias=True, scale=2.5, shared_I=2048,
                               wdt="fp8", seed=2000, weight_seed=2000),
    "r1_decode_mxfp4": MoEConfig("r1_decode_mxfp4", T=128, H=7168, E=256, k=8, I=2048,
                                 score="sigmoid", use_bias=True, scale=2.5, shared_I=2048,
                                 wdt="mxfp4", seed=2000, weight_seed=2000),
    # W8A8: r1_decode and r1_prefill with INT8 expert weights (128 x 128 blocks, fp32
    # scales amax/127) and INT8 activations (1 x 128 blocks) on the INT8 matrix units: same
    # seeds, so the same router and routing as the bf16 layers
    "r1_decode_int8": MoEConfig("r1_decode_int8", T=128, H=7168, E=256, k=8, I=2048,
                                score="sigmoid", use_bias=True, scale=2.5, shared_I=2048,
                                wdt="int8", seed=2000, weight_seed=2000),
    "r1_prefill_int8": MoEConfig("r1_prefill_int8", T=8192, H=7168, E=256, k=8, I=2048,
                                 score="sigmoid", use_bias=True, scale=2.5, shared_I=2048,
                                 wdt="int8", seed=3000, weight_seed=2000, zipf_s=1.1,
                                 zipf_gamma=PREFILL_ZIPF_GAMMA),
    # one GPU's expert-parallel share with both GEMM operands in MXFP4 (W4A4): ep32_mxfp4's
    # weights, rows and loads, with the activations quantised to MXFP4 inside
    "ep32_w4a4": MoEConfig("ep32_w4a4", T=16384, H=7168, E=32, k=1, I=2048, score="none",
                           act="bf16", wdt="mxfp4a4", out="bf16", seed=5000, weight_seed=5000,
                           dirichlet_alpha=0.5),
}

ORDER = ["tiny_fp32", "r1_decode", "r1_prefill", "e384_fp8", "ep32_mxfp4"]
