"""Builds libmoe.so (the C-ABI MoE layer library) for gfx950 with hipcc, in-tree."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe.so")

SOURCES = ["moe_api.hip", "route.hip", "permute.hip", "grouped_ffn.hip", "ffn_stream.hip",
           "ffn_tiled.hip", "ffn_fp8.hip", "combine.hip", "balance.hip", "ffn_w4a4.hip", "ffn_generic.hip",
           "probe.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False, extra=None, out: str = LIB) -> str:
    cmd = ["hipcc", *FLAGS, *(extra or []), *[os.path.join(CSRC, s) for s in SOURCES], "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("libmoe build failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    if verbose:
        print(" ".join(cmd))
        msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
        if msg.strip():
            print(msg)
    return out


if __name__ == "__main__":
    build(verbose=True)
