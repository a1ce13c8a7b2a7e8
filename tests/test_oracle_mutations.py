"""The oracle's pins have teeth: each plausible mistake below, planted in a copy of the oracle,
makes at least one CPU pin fail (CPU only; each case runs the pin files in a subprocess with
the mutated copy first on the import path).

The mistakes: a dropped or unquantised shared expert, a router fed quantised activations, a
combine without the shared term or with the permutation the wrong way round, h re-quantised
from its float64 value instead of its fp32 value (fp8, MXFP4, INT8), no re-quantisation of
h, and unquantised INT8 activations.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["test_oracle.py", "test_oracle_composition.py", "test_oracle_int8.py"]

MUTATIONS = {
    "shared_dropped": [
        ("        out += expert_ffn(a, w13, w2, requant_h=requant)", "        pass")],
    "shared_unquantised": [
        ("        out += expert_ffn(a, w13, w2, requant_h=requant)",
         "        out += expert_ffn(xs, w13, w2, requant_h=requant)")],
    "router_on_quantised_x": [
        ("        r = route(x64, decode_act(cfg.act, prob.wr)",
         "        r = route(quantise_rows_e4m3(x64.astype(np.float32))[2] "
         "if cfg.wdt in ('fp8', 'int8', 'mxfp4a4') else x64, decode_act(cfg.act, prob.wr)")],
    "combine_without_shared": [("        out = out + shared64", "        out = out")],
    "combine_permutation_inverted": [
        ("    rows = y64[np.asarray(inv_perm, np.int64).reshape(T, k)]",
         "    rows = y64[np.argsort(np.asarray(inv_perm, np.int64)).reshape(T, k)]")],
    "fp8_requant_from_float64": [
        ("        _, _, h = quantise_rows_e4m3(h.astype(np.float32))",
         "        _, _, h = quantise_rows_e4m3(h)"),
        ("    v = np.asarray(v32, np.float32)\n    R, C = v.shape",
         "    v = np.asarray(v32, np.float64)\n    R, C = v.shape")],
    "mxfp4_requant_from_float64": [
        ("        _, _, h = quantise_rows_mxfp4(h.astype(np.float32))",
         "        _, _, h = quantise_rows_mxfp4(h)"),
        ("    v = np.asarray(v32, np.float32).astype(np.float64)\n    R, C = v.shape\n"
         "    vb = v.reshape(R, C // block, block)\n    amax = np.abs(vb).max(axis=2)\n    _, ex",
         "    v = np.asarray(v32, np.float64)\n    R, C = v.shape\n"
         "    vb = v.reshape(R, C // block, block)\n    amax = np.abs(vb).max(axis=2)\n    _, ex")],
    "int8_requant_from_float64": [
        ("        _, _, h = quantise_rows_int8(h.astype(np.float32))",
         "        _, _, h = quantise_rows_int8(h)"),
        ("    s = np.where(amax == 0, np.float32(1.0), (amax / np.float32(127.0)).astype(np.float32))\n"
         "    s = s.astype(np.float32)\n    scaled = (vb / s[:, :, None]).astype(np.float32)",
         "    s = np.where(amax == 0, 1.0, amax.astype(np.float64) / 127.0)\n"
         "    scaled = vb.astype(np.float64) / s[:, :, None]")],
    "int8_h_not_requantised": [
        ("        _, _, h = quantise_rows_int8(h.astype(np.float32))", "        pass")],
    "int8_activations_unquantised": [
        ("        _, _, a = quantise_rows_int8(xs.astype(np.float32))", "        a = xs")],
}


def _run_pins(tmp_path, edits):
    """Copy the oracle to tmp_path, apply the edits, run the pin files against the copy."""
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle")
    path = tmp_path / "oracle" / "moe_oracle.py"
    src = path.read_text()
    for old, new in edits:
        assert old in src, old
        src = src.replace(old, new, 1)
    # mark the copy, so that the run can show which oracle it imported
    path.write_text(src + "\nMUTATED_COPY = True\n")
    env = dict(os.environ, PYTHONPATH=f"{tmp_path}{os.pathsep}{ROOT}")
    # run from tmp_path so that the repository root does not come first on sys.path
    check = subprocess.run([sys.executable, "-c", "import oracle.moe_oracle as m; print(m.MUTATED_COPY)"],
                           cwd=tmp_path, env=env, capture_output=True, text=True, timeout=120)
    assert check.stdout.strip() == "True", check.stderr
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                           *[os.path.join(ROOT, "tests", p) for p in PINS]],
                          cwd=tmp_path, env=env, capture_output=True, text=True, timeout=300)


@pytest.mark.slow
def test_unmodified_copy_passes(tmp_path):
    r = _run_pins(tmp_path, [])
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_fails_a_pin(name, tmp_path):
    r = _run_pins(tmp_path, MUTATIONS[name])
    assert r.returncode == 1 and " failed" in r.stdout, (name, r.stdout[-2000:])
