"""Benchmark of the MI355X MoE layer: one JSON line on stdout.

A step is one moe_layer_forward (route, permute, grouped SwiGLU FFN of the routed and the
shared experts, combine) over one batch of the workload, with inputs and weights resident
in HBM; for the pre-routed workload (ep32_mxfp4: one GPU's share of received rows) it is
one moe_rows_forward (permute, grouped FFN, combine). Default workload: the DeepSeek-R1-shaped decode layer (T=128 tokens, H=7168, 256
routed experts, top-8, sigmoid scores with a selection-only bias, weights renormalised
and scaled by 2.5, one shared expert, I=2048, bf16).

Besides layer tokens/s the line carries:
  roofline      the dominant kernel (grouped gate/up + SwiGLU) timed with HIP events
                recorded by the library around it on the stream it runs on; its
                algorithmic bytes (touched experts' gate/up weights + activation rows read
                + h written) per launch over its average duration, against 8 TB/s HBM;
                also against the device's measured peak of the same bound (a streaming
                read, or a dense MFMA loop, run by the library's measurement probes in the
                same process): measured_peak and frac_of_measured; for an MFMA-bound launch
                also against min(MFMA peak, AI x HBM peak): attainable, frac_of_attainable.
  cpu_baseline  the CPU oracle (float64 numpy) on a bounded sample of the same batch
                (the first few tokens; routing covers all tokens), tokens/s.
Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "MoE layer tokens/s + grouped-GEMM % of HBM/MFMA peak, 256e top-8 H=7168 bf16"
# a decode workload and the prefill-sized batch of the same layer, timed after it
PREFILL_OF = {"r1_decode": "r1_prefill"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="r1_decode")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline leg")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill-sized batch timed after a decode workload")
    ap.add_argument("--overlap", action="store_true",
                    help="also time the step with the shared expert on a side stream")
    ap.add_argument("--split", action="store_true",
                    help="also time moe_layer_forward_split (groups of few rows on a second "
                         "stream), with and without disjoint CU masks, on the named workload "
                         "(the prefill batch timed after a decode workload always gets it)")
    ap.add_argument("--cpu-tokens", type=int, default=72,
                    help="tokens of the batch the CPU oracle leg computes (about 10 s of CPU work)")
    ap.add_argument("--no-measured-peaks", dest="measured_peaks", action="store_false",
                    help="skip the streaming-read and MFMA-loop probes of the device's rates")
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="pre-routed workloads (weights under 1 GB, not many times the 256 MB "
                         "Infinity Cache): before each timed step write this many MiB of "
                         "device memory, outside the timing, so that no weights stay cached "
                         "from the step before; 0 times the steps back to back")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, run 3 plain device copies of this many MiB (a known-size "
                         "reference kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(cfg, host, n_tokens):
    """The oracle, as is, on the first n_tokens tokens of the batch (routing of all T)."""
    import numpy as np

    import oracle as O

    try:
        from threadpoolctl import threadpool_info

        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    tokens = list(range(min(n_tokens, cfg.T)))

    class Cached:
        """The sample's expert weights generated up front, so the timed region is oracle work."""

        def __init__(self, bank, experts):
            self.fmt = bank.fmt
            self._13 = {e: bank.w13(e) for e in experts}
            self._2 = {e: bank.w2(e) for e in experts}

        def w13(self, e):
            return self._13[e]

        def w2(self, e):
            return self._2[e]

    if cfg.routed:
        r = O.route(O.decode_act(cfg.act, host.x), O.decode_act(cfg.act, host.wr), host.bias, cfg.k,
                    cfg.score, cfg.scale)
        used = sorted(set(np.unique(r["topk_idx"][tokens]).tolist()))
    else:
        used = sorted(set(np.unique(host.topk_idx[tokens]).tolist()))
    log(f"cpu baseline: generating {len(used)} experts for {len(tokens)} tokens")
    host.routed = Cached(host.routed, used)
    if host.shared is not None:
        host.shared = Cached(host.shared, [0])
    t0 = time.perf_counter()
    res = O.layer_forward(host, tokens=tokens)
    dt = time.perf_counter() - t0
    assert res["out"].shape[0] == len(tokens)
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                         None)
    except OSError:  # pragma: no cover
        pass
    return {"value": len(tokens) / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": model,
            "sample": f"{len(tokens)} of {cfg.T} tokens of the same batch (routing of all {cfg.T} "
                      f"tokens, {len(used)} routed experts + shared expert FFNs in float64), "
                      f"{dt:.1f} s"}


# bytes per stored element (block scales included) of each storage format
ELEM_BYTES = {"f32": 4.0, "bf16": 2.0, "fp8": 1.0 + 4.0 / (128 * 128), "mxfp4": 0.5 + 1.0 / 32,
              "mxfp4a4": 0.5 + 1.0 / 32, "int8": 1.0 + 4.0 / (128 * 128)}
# dense MFMA peak (TFLOP/s) of the product each weight format is computed with: MXFP4 weights
# are decoded to bf16 in registers and multiplied on the bf16 MFMA
MFMA_PEAK = {"f32": 157.3, "bf16": BF16_PEAK_TFLOPS, "fp8": 5000.0, "mxfp4": BF16_PEAK_TFLOPS,
             "mxfp4a4": 10100.0, "int8": 5000.0}   # INT8: dense int8 TOP/s


def ffn_accounting(cfg, touched):
    """Algorithmic HBM bytes and flops of the grouped gate/up (+SwiGLU) and down launches:
    every touched expert's weights read once, every routed/shared row's input read once and
    its output written once; which of HBM or MFMA bounds each launch; the kernel the library
    picks for it (fp8: k_fp8; bf16 and fp32 with H or I not a multiple of 64: the plain
    dot-product kernels; bf16 and MXFP4 with more than 32 routed rows per expert on average:
    k_tiled2; otherwise the streaming kernels)."""
    T, H, I, Is, k = cfg.T, cfg.H, cfg.I, cfg.shared_I, cfg.k
    rows_r = T * k if cfg.routed else T
    rows = rows_r + (T if Is else 0)
    wb = ELEM_BYTES[cfg.wdt]
    q8 = 1.0 + 4.0 / 128          # an E4M3 code plus its share of a 1 x 128 fp32 scale
    q4 = 0.5 + 1.0 / 32           # an E2M1 code plus its share of a 1 x 32 E8M0 scale
    q8w = cfg.wdt in ("fp8", "int8")   # 8-bit codes with a 1 x 128 fp32 scale
    xb = q8 if q8w else (q4 if cfg.wdt == "mxfp4a4" else ELEM_BYTES[cfg.act])
    hb = q8 if q8w else (q4 if cfg.wdt == "mxfp4a4" else (4.0 if cfg.wdt == "f32" else 2.0))
    h_elems = rows_r * I + (T * Is if Is else 0)
    w13 = (touched * 2 * I * H + (2 * Is * H if Is else 0)) * wb
    w2 = (touched * I * H + (Is * H if Is else 0)) * wb
    fl_gu = 2.0 * (rows_r * H * 2 * I + (T * H * 2 * Is if Is else 0))
    fl_dn = 2.0 * (rows_r * I * H + (T * Is * H if Is else 0))
    if cfg.wdt == "fp8":
        kgu, kdn = "k_fp8<gate/up>", "k_fp8<down>"
    elif cfg.wdt == "int8":
        kgu, kdn = "k_fp8<gate/up, INT8>", "k_fp8<down, INT8>"
    elif cfg.wdt == "mxfp4" and rows_r <= 32 * cfg.E and H % 512 == 0 and I % 512 == 0:
        kgu, kdn = "k_gateup_stream_mx", "k_down_stream_mx"
    elif cfg.wdt == "mxfp4":
        kgu, kdn = "k_tiled2<gate/up, MXFP4>", "k_tiled2<down, MXFP4>"
    elif cfg.wdt == "mxfp4a4":
        kgu, kdn = "k_w4a4<gate/up>", "k_w4a4<down>"
    elif cfg.wdt in ("bf16", "f32") and (H % 64 or I % 64 or Is % 64):
        kgu, kdn = "k_gateup_generic", "k_down_generic"
    elif cfg.wdt == "bf16" and rows_r > 32 * cfg.E:
        kgu, kdn = "k_tiled2<gate/up>", "k_tiled2<down>"
    else:
        kgu, kdn = "k_gateup_stream", "k_down_stream"
    peak = MFMA_PEAK[cfg.wdt]

    def launch(nbytes, flops, kernel):
        bound = "mfma" if flops / (peak * 1e12) > nbytes / (HBM_PEAK_GBS * 1e9) else "hbm"
        frac_fn = ((lambda t: nbytes / t / 1e9 / HBM_PEAK_GBS) if bound == "hbm"
                   else (lambda t: flops / t / 1e12 / peak))
        return {"bytes": nbytes, "flops": flops, "bound": bound, "kernel": kernel,
                "mfma_peak": peak, "frac_fn": frac_fn}

    return {
        "gate_up": launch(w13 + rows * H * xb + h_elems * hb, fl_gu, kgu),
        # expert outputs: fp32 for bf16/fp32 banks, bf16 for the quantised formats
        "down": launch(w2 + h_elems * hb + rows * H * (4.0 if cfg.wdt in ("bf16", "f32") else 2.0),
                       fl_dn, kdn),
        # router weights + x read by the router (routed layers), output written by the combine
        "other_bytes": ((cfg.E * H + T * H) * ELEM_BYTES[cfg.act] if cfg.routed else 0)
        + T * H * ELEM_BYTES[cfg.out],
        "router_flops": 2.0 * T * cfg.E * H if cfg.routed else 0.0,
    }


def measured_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter
    summary (profiles/traffic_<workload>.json: FETCH_SIZE and WRITE_SIZE scaled by a plain
    copy of known size), or None when absent or taken on kernel sources that have changed."""
    import hashlib

    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest()[:16] != rec["source_sha256_16"]:
        return None
    return rec["traffic_bytes"]


def percentile(v, q):
    import numpy as np

    return float(np.percentile(np.asarray(v, np.float64), q))


# the matrix-core product each weight format is computed with (MXFP4 weights are decoded to
# bf16 and multiplied on the bf16 MFMA), as moe_probe_mfma names it
PROBE_DTYPE = {"bf16": "bf16", "fp8": "fp8", "int8": "int8", "mxfp4": "bf16",
               "mxfp4a4": "mxfp4a4"}


def measured_peaks(dtypes, read_gib=4):
    """The device's measured rates, for fractions against measured peaks beside the
    datasheet ones: one non-temporal streaming read of read_gib GiB (moe_probe_hbm_read)
    and dense MFMA loops on register operands at four wavefronts a SIMD on every CU
    (moe_probe_mfma), each timed with events on the stream it runs on; the best of five
    runs after a warm-up."""
    import torch

    import mixture_experts_layer_04_amd as moe

    stream = torch.cuda.current_stream()
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best_s(fn):
        fn()
        torch.cuda.synchronize()
        t = []
        for _ in range(5):
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            t.append(a.elapsed_time(b) / 1e3)
        return min(t)

    buf = torch.empty(read_gib << 30, dtype=torch.uint8, device="cuda")
    res = {"hbm_read_GBs": buf.numel() / best_s(lambda: moe.moe_probe_hbm_read(buf, sink)) / 1e9}
    del buf
    for dt in sorted(set(dtypes)):
        iters = 20000
        flops = moe.moe_probe_mfma(dt, iters, sink)  # the same count every launch
        res[f"{dt}_mfma_TFLOPs"] = flops / best_s(lambda: moe.moe_probe_mfma(dt, iters, sink)) / 1e12
    log("measured peaks: " + ", ".join(f"{k}={v:.1f}" for k, v in res.items()))
    return res


def add_measured(roofline, peaks, wdt):
    """Fractions of the dominant kernel against the measured peak of its bound and, for an
    MFMA-bound launch, against the attainable min(peak, AI x HBM peak)."""
    if roofline["bound"] == "hbm":
        m = peaks["hbm_read_GBs"]
    else:
        m = peaks[f"{PROBE_DTYPE[wdt]}_mfma_TFLOPs"]
        ai = roofline["algorithmic_flops_per_launch"] / roofline["algorithmic_bytes_per_launch"]
        att = min(roofline["peak"], ai * HBM_PEAK_GBS / 1e3)
        roofline["attainable"] = att
        roofline["frac_of_attainable"] = roofline["achieved"] / att
    roofline["measured_peak"] = m
    roofline["frac_of_measured"] = roofline["achieved"] / m


def run_workload(cfg, dev, args, overlap=False):
    """Times one workload: K plain steps between two events (ms/step), then K steps of the
    same launches with the library's stage events (per-stage means, and the median and
    p10/p90 of the per-step times). Returns a dict of the measurements."""
    import numpy as np
    import torch

    import mixture_experts_layer_04_amd as moe

    T, H, E = cfg.T, cfg.H, cfg.E
    odt = torch.float32 if cfg.out == "f32" else torch.bfloat16
    out = torch.empty((T, H), dtype=odt, device="cuda")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    ev = moe.StageEvents()
    stream = torch.cuda.current_stream()
    layer = None
    if cfg.routed:
        # a step: the whole layer (route, permute, grouped FFN incl. shared expert, combine)
        layer = moe.MoELayer.from_problem(cfg, dev)

        def step():
            layer.forward(dev.x, out, counts=counts)

        def timed_step():
            moe.moe_layer_forward_timed(layer.desc, dev.x, out, layer.ws, ev, counts=counts)
    else:
        # pre-routed rows (one GPU's expert-parallel share): permute, grouped FFN, combine
        bank = moe.Experts.from_bank(dev.routed)
        ws = moe.workspace(moe.moe_rows_workspace_size(bank, moe.DTYPES[cfg.act], T))
        row_e, row_w = dev.topk_idx.view(-1), dev.topk_w.view(-1)
        counts.copy_(torch.bincount(row_e.long(), minlength=E).int())

        def step():
            moe.moe_rows_forward(bank, dev.x, row_e, row_w, out, ws)

        def timed_step():
            moe.moe_rows_forward_timed(bank, dev.x, row_e, row_w, out, ws, ev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"{cfg.name}: warmup done ({args.warmup} steps)")

    # the routed workloads' weights (17-23 GB) are far beyond the 256 MB Infinity Cache; a
    # pre-routed share's (0.7 GB) is not, so each of its steps starts after a large write
    flush = None
    if not cfg.routed and args.flush_mib > 0:
        flush = torch.empty(args.flush_mib << 20, dtype=torch.uint8, device="cuda")

    def evict():
        if flush is not None:
            flush.fill_(1)
            torch.cuda.synchronize()

    # timed region: K plain steps (back to back, or each after the flush, outside its events)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    if flush is None:
        start.record(stream)
        for _ in range(args.steps):
            step()
        stop.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(stop) / args.steps
    else:
        tot = 0.0
        for _ in range(args.steps):
            evict()
            start.record(stream)
            step()
            stop.record(stream)
            torch.cuda.synchronize()
            tot += start.elapsed_time(stop)
        ms = tot / args.steps
    log(f"{cfg.name}: timed {args.steps} steps: {ms:.4f} ms/step"
        + (f" (each after a {args.flush_mib} MiB cache flush)" if flush is not None else ""))

    # per-stage times of the same launches, from events the library records on its stream
    stage = {s_: [] for s_ in moe.STAGES}
    per_step = []
    for _ in range(args.steps):
        evict()
        timed_step()
        torch.cuda.synchronize()
        st = ev.elapsed_ms()
        for s_, v in st.items():
            stage[s_].append(v)
        per_step.append(sum(st.values()))
    stage_ms = {s_: float(np.mean(v)) for s_, v in stage.items()}
    log(f"{cfg.name}: stage ms: " + ", ".join(f"{s_}={v:.4f}" for s_, v in stage_ms.items()))

    # the same step with the shared expert on a side stream beside the routed experts
    ovl_ms = None
    if overlap and cfg.routed and cfg.shared_I:
        fj = moe.ForkJoin()
        for _ in range(args.warmup):
            layer.forward_overlap(dev.x, out, fj, counts=counts)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(args.steps):
            layer.forward_overlap(dev.x, out, fj, counts=counts)
        stop.record(stream)
        torch.cuda.synchronize()
        ovl_ms = start.elapsed_time(stop) / args.steps
        log(f"{cfg.name}: overlapped shared expert: {ovl_ms:.4f} ms/step")

    cnt = counts.cpu().numpy()
    touched = int((cnt > 0).sum())
    acct = ffn_accounting(cfg, touched)
    g = acct["gate_up"]
    gu_s = stage_ms["gate_up"] / 1e3
    if g["bound"] == "hbm":
        achieved, peak, unit = g["bytes"] / gu_s / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        achieved, peak, unit = g["flops"] / gu_s / 1e12, g["mfma_peak"], "TFLOP/s"
    layer_bytes = acct["gate_up"]["bytes"] + acct["down"]["bytes"] + acct["other_bytes"]
    layer_flops = acct["gate_up"]["flops"] + acct["down"]["flops"] + acct["router_flops"]
    ffn_s = (stage_ms["gate_up"] + stage_ms["down"]) / 1e3
    ffn_flops = acct["gate_up"]["flops"] + acct["down"]["flops"]
    return {
        "ms": ms, "stage_ms": stage_ms, "touched": touched, "counts": counts,
        "cache_flush_mib": args.flush_mib if flush is not None else 0,
        "step_ms_p10_p50_p90": [percentile(per_step, q) for q in (10, 50, 90)],
        "ovl_ms": ovl_ms,
        "layer_bytes": layer_bytes, "layer_flops": layer_flops,
        "down_frac": acct["down"]["frac_fn"](stage_ms["down"] / 1e3),
        "ffn_tflops": ffn_flops / ffn_s / 1e12,
        "ffn_mfma_frac": ffn_flops / ffn_s / 1e12 / acct["gate_up"]["mfma_peak"],
        "roofline": {"bound": g["bound"], "kernel": f"grouped gate/up + SwiGLU ({g['kernel']})",
                     "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
                     "traffic": measured_traffic(cfg.name),
                     "algorithmic_bytes_per_launch": g["bytes"],
                     "algorithmic_flops_per_launch": g["flops"],
                     "avg_launch_ms": stage_ms["gate_up"]},
    }


def time_split(cfg, dev, args):
    """ms/step of moe_layer_forward_split for a few cold-row thresholds, on two plain streams
    and on streams with disjoint CU masks (a quarter of the CUs for the cold groups); host
    clock around K steps on the split streams, which torch's events do not see."""
    import torch

    import mixture_experts_layer_04_amd as moe

    layer = moe.MoELayer.from_problem(cfg, dev)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    res = {}
    for masked in (False, True):
        ss = moe.SplitStreams(*moe.cu_masks(n_cu)) if masked else moe.SplitStreams()
        for cold_max in (32, 64, 128):
            for _ in range(args.warmup):
                moe.moe_layer_forward_split(layer.desc, dev.x, out, layer.ws, ss, cold_max)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                moe.moe_layer_forward_split(layer.desc, dev.x, out, layer.ws, ss, cold_max)
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) / args.steps * 1e3
            key = f"{'cu_masked' if masked else 'shared_cus'}_cold_le_{cold_max}"
            res[key] = ms
            log(f"{cfg.name}: split {key}: {ms:.4f} ms/step")
        del ss
    return res


def describe(cfg):
    return (f"{cfg.name}: T={cfg.T} H={cfg.H} E={cfg.E} top-{cfg.k} I={cfg.I} {cfg.score}"
            f"{' + selection bias' if cfg.use_bias else ''} scale {cfg.scale}"
            f"{', Zipf-skewed router' if cfg.zipf_s else ''}, "
            f"{'1 shared expert, ' if cfg.shared_I else ''}{cfg.wdt}")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(multi-GPU expert parallelism is not built)", file=sys.stderr)
        sys.exit(2)
    import torch

    import mixture_experts_layer_04_amd as moe
    from synth.configs import CONFIGS
    from synth.problem import device_problem, host_problem

    cfg = CONFIGS[args.workload]
    log(f"workload {cfg.name}: generating inputs on the device")
    host = host_problem(cfg)
    dev = device_problem(cfg, host=host)
    T = cfg.T
    r = run_workload(cfg, dev, args, overlap=args.overlap)
    split = time_split(cfg, dev, args) if args.split and cfg.routed and cfg.wdt == "bf16" else None

    # the selection-bias balancing step (not part of the forward step): its own timing
    bias_us = None
    if cfg.routed and cfg.use_bias:
        stream = torch.cuda.current_stream()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b = dev.bias.clone()
        reps = 200
        start.record(stream)
        for _ in range(reps):
            moe.moe_bias_update(r["counts"], 1e-3, b)
        stop.record(stream)
        torch.cuda.synchronize()
        bias_us = start.elapsed_time(stop) / reps * 1e3
        log(f"bias update: {bias_us:.2f} us per call")

    # the prefill-sized batch of the same layer (same expert banks, 64x the tokens, a skewed
    # router): the MFMA-bound half of the metric, measured in the same process
    prefill = None
    pname = PREFILL_OF.get(cfg.name)
    if pname and not args.no_prefill:
        pcfg = CONFIGS[pname]
        log(f"workload {pcfg.name}: generating activations and router on the device "
            f"(expert banks shared with {cfg.name})")
        pdev = device_problem(pcfg, banks_of=dev)
        p = run_workload(pcfg, pdev, args)
        psplit = time_split(pcfg, pdev, args)
        prefill = {"workload": describe(pcfg), "tokens": pcfg.T, "ms_per_step": p["ms"],
                   "ms_per_step_split": psplit,
                   "tokens_per_s": pcfg.T / (p["ms"] / 1e3), "experts_touched": p["touched"],
                   "stage_ms": {s_: round(v, 5) for s_, v in p["stage_ms"].items()},
                   "step_ms_p10_p50_p90": p["step_ms_p10_p50_p90"],
                   "grouped_ffn_tflops": p["ffn_tflops"],
                   "grouped_ffn_mfma_frac": p["ffn_mfma_frac"],
                   "down_frac": p["down_frac"],
                   "roofline": p["roofline"]}
        del pdev

    # measured peaks of the device (measurement probes), for fractions of measured peaks
    probes = [PROBE_DTYPE[c.wdt] for c in ([cfg] + ([CONFIGS[pname]] if prefill else []))
              if c.wdt in PROBE_DTYPE]
    if args.measured_peaks:
        peaks = measured_peaks(probes)
        add_measured(r["roofline"], peaks, cfg.wdt)
        if prefill:
            add_measured(prefill["roofline"], peaks, CONFIGS[pname].wdt)

    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy probe: 3 x {args.copy_probe_mib} MiB device copies")

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cfg, host, args.cpu_tokens)
        log(f"cpu baseline: {cpu['value']:.3f} tokens/s on {cpu['cores']} threads")

    ms = r["ms"]
    line = {
        "metric": METRIC,
        "value": T / (ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.wdt,
        "data": "synthetic (seeded Philox inputs; N(0,1) activations, N(0,0.02) weights)",
        "config": {"workload": describe(cfg),
                   "tokens": T, "experts_touched": r["touched"],
                   "stage_ms": {s_: round(v, 5) for s_, v in r["stage_ms"].items()},
                   "step_ms_p10_p50_p90": r["step_ms_p10_p50_p90"],
                   "cache_flush_mib_before_each_step": r["cache_flush_mib"],
                   "layer_algorithmic_bytes": r["layer_bytes"], "layer_flops": r["layer_flops"],
                   "layer_hbm_frac": r["layer_bytes"] / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                   "down_frac": r["down_frac"],
                   "bias_update_us": bias_us,
                   "ms_per_step_shared_overlapped": r["ovl_ms"],
                   "ms_per_step_split": split,
                   "prefill": prefill},
        "roofline": r["roofline"],
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
