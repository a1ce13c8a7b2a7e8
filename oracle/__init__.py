"""CPU oracle of the MoE layer (float64 numpy). Test infrastructure only: imported
by the test suite, the package smoke check and the benchmark's CPU-baseline leg,
never by the GPU library."""
from .moe_oracle import *  # noqa: F401,F403
