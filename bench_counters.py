"""Summarise rocprofv3 runs of bench.py into the text profiles kept under profiles/.

Input: one directory with a kernel-trace run `<W>_trace/` (and its stdout `<W>_trace.out`,
whose last line is bench.py's JSON line) and five counter runs `<W>_p1/` .. `<W>_p5/`, made
by these commands (from /tmp after `export TMPDIR=/tmp`; `<repo>` is the repository root):

    rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/<W>_trace -o run -- \
        python3 <repo>/bench.py --workload <W> --steps 20 --warmup 3 --no-cpu --no-prefill
    rocprofv3 --pmc <pass i counters> --output-format csv -d <dir>/<W>_p<i> -o run -- \
        python3 <repo>/bench.py --workload <W> --steps 2 --warmup 1 --no-cpu --no-prefill \
        --copy-probe-mib 1024

The counter passes are PASSES below. GRBM_GUI_ACTIVE is summed over the 8 XCDs, so divided
by 8 and by a dispatch's duration it is the average shader clock. SQ_VALU_MFMA_BUSY_CYCLES
is summed over the 1024 SIMDs. FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by
what they read for the three 1 GiB device copies that --copy-probe-mib adds.

    python bench_counters.py <dir> <W> <kernel substring> [<kernel substring> ...] \
        [--md profiles/<name>.md] [--traffic-json profiles/traffic_<W>.json --sources f ...]
"""
import argparse
import collections
import csv
import hashlib
import json
import os

ROOT = os.path.dirname(os.path.abspath(__file__))
N_XCD, N_SIMD = 8, 1024
PASSES = [
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F8 "
    "SQ_INSTS_MFMA SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_INSTS_VALU GRBM_GUI_ACTIVE",
    "SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_ACTIVE_INST_LDS SQ_WAIT_INST_LDS "
    "SQ_LDS_ADDR_CONFLICT SQ_INSTS_SALU GRBM_GUI_ACTIVE",
    "SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_VMEM "
    "SQ_ACTIVE_INST_MISC SQ_ACTIVE_INST_SCA SQ_INSTS_VMEM_RD GRBM_GUI_ACTIVE",
    "FETCH_SIZE TCC_HIT_sum GRBM_GUI_ACTIVE",
    "WRITE_SIZE TCC_MISS_sum GRBM_GUI_ACTIVE",
]
COPY = "__amd_rocclr_copyBuffer"


def copy_kib(path, counter):
    """Mean of the counter over the three large copies (other copies in the run are a few
    bytes: results read back by the tests' and bench's own code)."""
    v = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if COPY in r["Kernel_Name"] and r["Counter_Name"] == counter:
                v.append(float(r["Counter_Value"]))
    big = [x for x in v if x >= 0.5 * max(v)]
    return sum(big) / len(big)


def load_pass(path):
    """kernel name -> {counter: mean over dispatches}, plus mean duration (us) and the
    dispatch's resources (VGPRs, LDS, scratch)."""
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    dur = collections.defaultdict(dict)
    res = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            k = r["Kernel_Name"]
            vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
            dur[k][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            res[k] = {"vgpr": int(r["VGPR_Count"]), "agpr": int(r["Accum_VGPR_Count"]),
                      "lds": int(r["LDS_Block_Size"]), "scratch": int(r["Scratch_Size"])}
    out = {}
    for k, cs in vals.items():
        d = {c: sum(v) / len(v) for c, v in cs.items()}
        d["dur_us"] = sum(dur[k].values()) / len(dur[k])
        out[k] = (d, res[k])
    return out


def find(table, sub):
    ks = [k for k in table if sub in k]
    if not ks:
        raise SystemExit(f"no kernel matching {sub!r}")
    if len(set(ks)) > 1:
        ks.sort(key=len)
    return ks[0]


def short(name):
    name = name.replace("moe::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
    return name.split("(")[0]


def summarise(d, w, subs):
    passes = [load_pass(os.path.join(d, f"{w}_p{i + 1}", "run_counter_collection.csv"))
              for i in range(len(PASSES))]
    fetch_copy = copy_kib(os.path.join(d, f"{w}_p4", "run_counter_collection.csv"), "FETCH_SIZE")
    write_copy = copy_kib(os.path.join(d, f"{w}_p5", "run_counter_collection.csv"), "WRITE_SIZE")
    fscale, wscale = (1 << 20) / fetch_copy, (1 << 20) / write_copy   # KiB per GiB copied
    rows = []
    for sub in subs:
        c, dur = {}, []
        for p in passes:
            d, res = p[find(p, sub)]
            dur.append(d["dur_us"])
            for key, v in d.items():
                c.setdefault(key, v)
        name = find(passes[0], sub)
        # clock from pass 1's own GRBM_GUI_ACTIVE and duration
        p1 = passes[0][name][0]
        clock = p1["GRBM_GUI_ACTIVE"] / N_XCD / (p1["dur_us"] * 1e3)
        flops = c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 + c["SQ_INSTS_VALU_MFMA_MOPS_F8"] * 512
        hit = c["TCC_HIT_sum"] / max(1.0, c["TCC_HIT_sum"] + c["TCC_MISS_sum"])
        rows.append({
            "kernel": short(name), "full_name": name, "resources": res,
            "dur_us_passes": dur, "clock_ghz": clock,
            "mfma_busy": c["SQ_VALU_MFMA_BUSY_CYCLES"] / (N_SIMD * p1["GRBM_GUI_ACTIVE"] / N_XCD),
            "mfma_insts": c["SQ_INSTS_MFMA"], "mfma_flops": flops,
            "valu_insts": c["SQ_INSTS_VALU"], "lds_insts": c["SQ_INSTS_LDS"],
            "lds_bank_conflict_frac": c["SQ_LDS_BANK_CONFLICT"] / max(1.0, c["SQ_LDS_IDX_ACTIVE"]),
            "wait_frac": c["SQ_WAIT_ANY"] / max(1.0, c["SQ_WAVE_CYCLES"]),
            "l2_hit": hit,
            "fetch_kib": c["FETCH_SIZE"], "write_kib": c["WRITE_SIZE"],
            "fetch_bytes": c["FETCH_SIZE"] * fscale * 1024, "write_bytes": c["WRITE_SIZE"] * wscale * 1024,
        })
    return rows, fscale, wscale


def kernel_stats(d, w, top=12):
    with open(os.path.join(d, f"{w}_trace", "run_kernel_stats.csv")) as f:
        return list(csv.DictReader(f))[:top]


def bench_line(path):
    with open(path) as f:
        lines = [ln for ln in f if ln.startswith("{")]
    return json.loads(lines[-1])


def markdown(d, w, subs, rows, fscale, wscale):
    line = bench_line(os.path.join(d, f"{w}_trace.out"))
    roof = line["roofline"]
    out = [f"# rocprofv3 summary: {rows[0]['kernel']} on {w}", "",
           f"Workload: {line['config']['workload']}.", "",
           "Commands (on one MI355X, from /tmp after `export TMPDIR=/tmp`; `<repo>` is the "
           "repository root, `<dir>` any output folder):", "",
           f"    rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/{w}_trace -o run -- "
           f"python3 <repo>/bench.py --workload {w} --steps 20 --warmup 3 --no-cpu --no-prefill"]
    for i, p in enumerate(PASSES):
        out.append(f"    rocprofv3 --pmc {p} --output-format csv -d <dir>/{w}_p{i + 1} -o run -- "
                   f"python3 <repo>/bench.py --workload {w} --steps 2 --warmup 1 --no-cpu "
                   f"--no-prefill --copy-probe-mib 1024")
    out += ["", "Summarised by `python3 <repo>/bench_counters.py <dir> " + w + " "
            + " ".join(f"'{x}'" for x in subs) + " --md <this file>`.", "",
            "## Kernel trace (--kernel-trace --stats)", "",
            "| kernel | calls | avg us | % of GPU time |", "|---|---|---|---|"]
    for r in kernel_stats(d, w):
        out.append(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} "
                   f"| {float(r['Percentage']):.2f} |")
    out += ["", "The synthetic-input fill kernels (k_normal_*, k_fp8_bank, k_int8_bank, "
            "k_mxfp4_bank, k_words) run once, before timing.", "",
            "## Dominant kernel against its roofline (bench.py's line in the trace run)", "",
            f"`{roof['kernel']}`: {roof['avg_launch_ms'] * 1e3:.1f} us a launch (HIP events "
            f"on its stream); {roof['algorithmic_bytes_per_launch']:.4g} B and "
            f"{roof['algorithmic_flops_per_launch']:.4g} flop algorithmic; bound {roof['bound']}: "
            f"{roof['achieved']:.1f} of {roof['peak']:.0f} {roof['unit']} = "
            f"**{roof['frac'] * 100:.1f}%**. Step: {line['ms_per_step']:.3f} ms; stages (ms): "
            + ", ".join(f"{k} {v:.3f}" for k, v in line["config"]["stage_ms"].items()) + ".", "",
            "## Counters per dispatch (means over the counter runs' dispatches)", "",
            f"FETCH_SIZE scale {fscale:.4f} and WRITE_SIZE scale {wscale:.4f}, from the 1 GiB "
            "copies of the same runs.", ""]
    keys = [("duration us (counter runs)", lambda r: " / ".join(f"{x:.0f}" for x in r["dur_us_passes"])),
            ("shader clock GHz", lambda r: f"{r['clock_ghz']:.2f}"),
            ("VGPRs / AGPRs / LDS B / scratch B", lambda r: "{vgpr} / {agpr} / {lds} / {scratch}".format(**r["resources"])),
            ("MFMA busy (of SIMD cycles)", lambda r: f"{r['mfma_busy'] * 100:.1f}%"),
            ("MFMA instructions", lambda r: f"{r['mfma_insts']:.4g}"),
            ("MFMA flops executed (MOPS x 512)", lambda r: f"{r['mfma_flops']:.4g}"),
            ("VALU instructions", lambda r: f"{r['valu_insts']:.4g}"),
            ("LDS instructions", lambda r: f"{r['lds_insts']:.4g}"),
            ("LDS bank-conflict cycles / LDS indexed-access cycles", lambda r: f"{r['lds_bank_conflict_frac'] * 100:.2f}%"),
            ("wave cycles waiting (SQ_WAIT_ANY / SQ_WAVE_CYCLES)", lambda r: f"{r['wait_frac'] * 100:.1f}%"),
            ("L2 hit rate", lambda r: f"{r['l2_hit'] * 100:.1f}%"),
            ("HBM read, scaled FETCH_SIZE", lambda r: f"{r['fetch_bytes'] / 1e9:.3f} GB"),
            ("HBM write, scaled WRITE_SIZE", lambda r: f"{r['write_bytes'] / 1e9:.3f} GB")]
    out.append("| | " + " | ".join(f"`{r['kernel']}`" for r in rows) + " |")
    out.append("|---|" + "---|" * len(rows))
    for label, fn in keys:
        out.append(f"| {label} | " + " | ".join(fn(r) for r in rows) + " |")
    return "\n".join(out) + "\n"


def traffic_json(w, row, fscale, wscale, sources):
    h = hashlib.sha256()
    for src in sources:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    return {"workload": w, "kernel": row["kernel"], "fetch_kib": row["fetch_kib"],
            "write_kib": row["write_kib"], "fetch_scale": fscale, "write_scale": wscale,
            "traffic_bytes": row["fetch_bytes"] + row["write_bytes"],
            "source_sha256_16": h.hexdigest()[:16], "sources": sources}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("dir")
    ap.add_argument("workload")
    ap.add_argument("kernels", nargs="+")
    ap.add_argument("--md")
    ap.add_argument("--traffic-json")
    ap.add_argument("--sources", nargs="*", default=[])
    a = ap.parse_args()
    rows, fs, ws = summarise(a.dir, a.workload, a.kernels)
    text = markdown(a.dir, a.workload, a.kernels, rows, fs, ws)
    if a.md:
        with open(a.md, "w") as f:
            f.write(text)
    else:
        print(text)
    if a.traffic_json:
        with open(a.traffic_json, "w") as f:
            json.dump(traffic_json(a.workload, rows[0], fs, ws, a.sources), f, indent=1)
            f.write("\n")


if __name__ == "__main__":
    main()
