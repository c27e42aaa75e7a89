"""Benchmark of one paged-attention step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config N] [--gpus 1]

A step is the whole hot path on one batch: slot derivation, KV scatter and
attention (host plan + split-K decode + merge + MFMA extend), run as the one
call with the KV update (pa_write_kv_attention; --separate: the three calls
pa_slot_mapping, pa_write_kv, pa_attention), with every input already in
HBM.  The default workload is the largest single-GPU configuration, the
mixed continuous-batching step with a 2048-token budget: 48 decode rows
(context U[256, 8192]) + a 512-token prefill chunk + a 1488-token chunk
after 1536 cached tokens; 32 q / 8 kv heads, head_dim 128, block 16, bf16,
40k-block pool.  It runs every kernel of the path.

Timing: each of the K timed steps starts with cold caches (a 1 GiB read
before the step, outside its HIP events, evicts L2 and the 256 MB Infinity
Cache); ms_per_step is their median, with p10 / p90.  The same K steps back
to back with warm caches are reported beside it.

Prints one JSON line: tokens/s (whole step), the dominant kernel against its
roofline (HIP events recorded around every launch on the stream it runs on,
over K more cold steps), the extend kernel against the bf16 MFMA peak when
the step has prefill rows, and the CPU oracle timed on this host on the same
workload.  Beside the published peaks, each roofline also gives its fraction
of what plain device work reaches in the same run (a 1 GiB read for HBM, the
vendor BLAS on an 8192^3 bf16 GEMM for MFMA; measured_ceilings).
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published
ELEM = {"f32": 4, "bf16": 2, "fp8": 1}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", type=int, default=3,
                    help="workload: 1-5 the reference configurations, 6 speculative verify, 7 long prefill")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time for the oracle baseline (0 disables it)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (for counter calibration) and exit")
    ap.add_argument("--traffic-ingest", nargs=4, metavar=("FETCH", "WRITE", "CAL_FETCH", "CAL_WRITE"),
                    help="turn four rocprofv3 --pmc output folders (FETCH_SIZE and WRITE_SIZE of "
                         "this workload, then of --copy-calibration) into the traffic record of "
                         "the dominant kernel under profiles/, and exit")
    ap.add_argument("--kernel", default="k_decode", help="kernel for --traffic-ingest / --counters-ingest")
    ap.add_argument("--trace-summary", nargs=2, metavar=("TRACE_DIR", "BENCH_OUT"),
                    help="turn a rocprofv3 --kernel-trace --stats folder of a bench.py run and that run's "
                         "output (its JSON line) into profiles/<kernel>_<workload>.md, and exit")
    ap.add_argument("--counters-ingest", nargs="+", metavar="DIR",
                    help="turn rocprofv3 --pmc output folders (one pass each) into the counter record "
                         "of --kernel on this workload under profiles/, and exit")
    ap.add_argument("--separate", action="store_true",
                    help="time the step as three calls (slot derivation, KV write, attention) "
                         "instead of the one call that includes the KV update")
    ap.add_argument("--compare", action="store_true",
                    help="also time the other form of the step (same pool and inputs)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured once into a HIP graph and replayed "
                         "(same batch every replay), and --graph-layers steps on as many pools "
                         "(the attention layers of one model step) eagerly and as one graph")
    ap.add_argument("--graph-layers", type=int, default=8,
                    help="layers (each its own pool and inputs) of the multi-layer graph timing")
    return ap.parse_args()


# Sources whose change invalidates a kernel's measured traffic.
KERNEL_SOURCES = {
    "k_decode": ["k_decode.hip", "k_decode_mfma.hip", "pa_device.h", "pa_internal.h", "pa_api.hip"],
    "k_extend": ["k_extend.hip", "pa_device.h", "pa_internal.h", "pa_api.hip"],
}
COPY_BYTES = 1 << 30


def source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "paged_kv_cache_pool_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_record_path(kernel, workload):
    return os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.md")


def _counter_per_dispatch(folder, counter, name_part):
    """Mean of `counter` over the dispatches whose kernel name contains name_part."""
    import csv
    import glob
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    vals = []
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]:
                    vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"{counter} for '{name_part}' not found under {folder}")
    return sum(vals) / len(vals), len(vals)


def _largest_dispatch(folder, counter):
    """Counter value of the dispatch reading/writing the most (the 1 GiB copy)."""
    import csv
    import glob
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    best = []
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    best.append(float(r["Counter_Value"]))
    best.sort()
    top = [v for v in best if v >= 0.5 * best[-1]]
    return sum(top) / len(top)


def traffic_ingest(a):
    """Write the traffic record: KiB per dispatch from FETCH_SIZE / WRITE_SIZE,
    each scaled by (bytes a plain 1 GiB copy moves) / (bytes the same counter
    reports for it)."""
    from paged_kv_cache_pool_amd import workloads as W
    fetch_dir, write_dir, cal_fetch_dir, cal_write_dir = a.traffic_ingest
    fetch_kib, n_f = _counter_per_dispatch(fetch_dir, "FETCH_SIZE", a.kernel)
    write_kib, n_w = _counter_per_dispatch(write_dir, "WRITE_SIZE", a.kernel)
    cal_fetch = COPY_BYTES / (1024.0 * _largest_dispatch(cal_fetch_dir, "FETCH_SIZE"))
    cal_write = COPY_BYTES / (1024.0 * _largest_dispatch(cal_write_dir, "WRITE_SIZE"))
    read_b = fetch_kib * 1024.0 * cal_fetch
    write_b = write_kib * 1024.0 * cal_write
    w = W.make(a.config, a.seed)
    rec = {"kernel": a.kernel, "workload": w.name, "source_sha": source_hash(a.kernel),
           "fetch_kib_per_dispatch": round(fetch_kib, 1), "write_kib_per_dispatch": round(write_kib, 1),
           "dispatches": [n_f, n_w], "copy_factor_fetch": round(cal_fetch, 4),
           "copy_factor_write": round(cal_write, 4), "hbm_bytes_read": round(read_b),
           "hbm_bytes_written": round(write_b), "hbm_bytes": round(read_b + write_b)}
    cmd = f"python bench.py --config {a.config} --steps 5 --warmup 2 --cpu-seconds 0"
    text = [f"# HBM traffic of {a.kernel}, workload {w.name}", "",
            "Counters (one pass each, on the MI355X, from the repository root):", "",
            "```",
            f"rocprofv3 --pmc FETCH_SIZE -d <fetch> -o run --output-format csv -- {cmd}",
            f"rocprofv3 --pmc WRITE_SIZE -d <write> -o run --output-format csv -- {cmd}",
            "rocprofv3 --pmc FETCH_SIZE -d <cal_fetch> -o run --output-format csv -- python bench.py --copy-calibration",
            "rocprofv3 --pmc WRITE_SIZE -d <cal_write> -o run --output-format csv -- python bench.py --copy-calibration",
            f"python bench.py --config {a.config} --kernel {a.kernel} --traffic-ingest <fetch> <write> <cal_fetch> <cal_write>",
            "```", "",
            f"FETCH_SIZE {fetch_kib:.1f} KiB and WRITE_SIZE {write_kib:.1f} KiB per dispatch "
            f"(mean of {n_f} / {n_w} dispatches).  A plain copy of {COPY_BYTES} bytes reads "
            f"{cal_fetch:.3f}x and writes {cal_write:.3f}x what the counters report, so the "
            f"kernel moves {read_b / 1e6:.1f} MB read + {write_b / 1e6:.1f} MB written per launch.",
            "bench.py reports this as roofline.traffic while the kernel's sources hash to "
            "source_sha below.", "", "```json", json.dumps(rec), "```", ""]
    path = traffic_record_path(a.kernel, w.name)
    with open(path, "w") as fh:
        fh.write("\n".join(text))
    print(json.dumps(rec), flush=True)


def counters_ingest(a):
    """Write the counter record of a kernel on a workload: the mean per
    dispatch of every counter found in the given --pmc passes, the kernel's
    mean duration from the same runs, and the derived figures:
    * MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 * 1024):
      the busy counter is summed over all 1024 SIMDs (32 cycles per
      32x32x16 MFMA), and GRBM_GUI_ACTIVE as reported is summed over the 8
      XCDs, each counting its own active cycles, so GRBM_GUI_ACTIVE / 8 is a
      SIMD's cycles during the dispatch;
    * clock = GRBM_GUI_ACTIVE / 8 / the dispatch's duration;
    * wave wait share = SQ_WAIT_ANY / SQ_WAVE_CYCLES, and busy-issue share =
      SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (waves that cannot issue)."""
    import csv
    import glob
    from paged_kv_cache_pool_amd import workloads as W
    vals, durs = {}, []
    for folder in a.counters_ingest:
        files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {folder}")
        for f in files:
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if a.kernel in r["Kernel_Name"]:
                        vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                        if "End_Timestamp" in r and r.get("Start_Timestamp"):
                            durs.append(float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    if not vals:
        raise SystemExit(f"no counters for '{a.kernel}'")
    mean = {k: sum(v) / len(v) for k, v in vals.items()}
    n = {k: len(v) for k, v in vals.items()}
    simds, xcds = 4 * 256, 8
    derived = {}
    dur_us = sum(durs) / len(durs) / 1e3 if durs else None
    if dur_us:
        derived["duration_us"] = dur_us
    if "GRBM_GUI_ACTIVE" in mean and dur_us:
        derived["clock_ghz"] = mean["GRBM_GUI_ACTIVE"] / xcds / (dur_us * 1e3)
    if "SQ_VALU_MFMA_BUSY_CYCLES" in mean and "GRBM_GUI_ACTIVE" in mean:
        derived["mfma_busy"] = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (mean["GRBM_GUI_ACTIVE"] / xcds * simds)
    if "SQ_INSTS_MFMA" in mean:
        derived["mfma_flops"] = mean["SQ_INSTS_MFMA"] * 32 * 32 * 16 * 2
    if "SQ_WAIT_ANY" in mean and "SQ_WAVE_CYCLES" in mean:
        derived["wave_wait_share"] = mean["SQ_WAIT_ANY"] / mean["SQ_WAVE_CYCLES"]
    if "SQ_WAIT_INST_ANY" in mean and "SQ_WAVE_CYCLES" in mean:
        derived["wave_no_issue_share"] = mean["SQ_WAIT_INST_ANY"] / mean["SQ_WAVE_CYCLES"]
    if "SQ_INSTS_LDS" in mean and "SQ_INSTS_VALU" in mean:
        derived["lds_per_valu"] = mean["SQ_INSTS_LDS"] / mean["SQ_INSTS_VALU"]
    w = W.make(a.config, a.seed)
    src_kernel = "k_extend" if a.kernel in ("k_extend_wide", "k_extend") else "k_decode"
    rec = {"kernel": a.kernel, "workload": w.name, "source_sha": source_hash(src_kernel),
           "counters_mean_per_dispatch": {k: round(v, 1) for k, v in sorted(mean.items())},
           "dispatches": n, "derived": {k: round(v, 4) for k, v in derived.items()}}
    cmd = f"python bench.py --config {a.config} --steps 5 --warmup 2 --cpu-seconds 0"
    text = [f"# Hardware counters of {a.kernel}, workload {w.name}", "",
            "One rocprofv3 --pmc pass per counter group, on the MI355X, from the repository root:", "",
            "```",
            f"rocprofv3 --pmc <counters of one pass> -d <pass folder> -o run --output-format csv -- {cmd}",
            f"python bench.py --config {a.config} --kernel {a.kernel} --counters-ingest <pass folders>",
            "```", "",
            "Derived: MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs) (the "
            "busy counter is summed over the SIMDs, GRBM_GUI_ACTIVE over the XCDs); clock = GRBM_GUI_ACTIVE "
            "/ 8 / duration; mfma_flops = SQ_INSTS_MFMA x 32768 (32x32x16 MFMAs); wave wait share = "
            "SQ_WAIT_ANY / SQ_WAVE_CYCLES; no-issue share = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES.",
            "The record holds the hash of the kernel's sources it was taken on.", "",
            "| counter | mean per dispatch |", "|---|---|"]
    text += [f"| {k} | {v:,.0f} |" for k, v in sorted(mean.items())]
    text += ["", "| derived | value |", "|---|---|"]
    text += [f"| {k} | {v:.4f} |" for k, v in derived.items()]
    text += ["", "```json", json.dumps(rec), "```", ""]
    path = os.path.join(ROOT, "profiles", f"counters_{a.kernel}_{w.name}.md")
    with open(path, "w") as fh:
        fh.write("\n".join(text))
    print(json.dumps(rec), flush=True)


def trace_summary(a):
    """Summary of a traced bench.py run: rocprofv3's per-kernel statistics over
    every launch, the average over the launches of the cold profiled pass
    (bench.py's roofline pass: launches W + K .. W + 2K - 1 of each step
    kernel), and the run's own JSON line."""
    import csv
    trace_dir, bench_out = a.trace_summary
    res = None
    with open(bench_out) as fh:
        for line in fh:
            if line.startswith("{") and '"metric"' in line:
                res = json.loads(line)
    if res is None:
        raise SystemExit(f"no JSON line in {bench_out}")
    stats = list(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_stats.csv"))))
    trace = list(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_trace.csv"))))
    W_, K_ = res["warmup"], res["steps"]
    by_kernel = {}
    for r in sorted(trace, key=lambda r: int(r["Start_Timestamp"])):
        by_kernel.setdefault(r["Kernel_Name"], []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    wl = res["config"]["workload"]
    dom = res["roofline"]["kernel"]
    cmd = (f"rocprofv3 --kernel-trace --stats -d <trace_dir> -o run --output-format csv -- python3 bench.py "
           f"--config {a.config} --steps {K_} --warmup {W_} --cpu-seconds 0 > <bench_out>")
    text = [f"# Kernel trace of one step of workload {wl} (seed {res['config']['seed']}), "
            f"{res['step_form']}", "",
            "Commands (repository root on the MI355X box):", "", "```", cmd,
            f"python bench.py --config {a.config} --trace-summary <trace_dir> <bench_out>", "```", "",
            f"The run does {W_} warm-up steps, then {K_} cold timed steps, {K_} cold steps with the "
            f"library's per-launch HIP events (the roofline pass), then {K_} warm steps: "
            f"{W_ + 3 * K_} launches of each kernel of the step.  A cold step starts after a 1 GiB read "
            "that evicts L2 and the Infinity Cache.", "",
            "| kernel | launches | avg us (all) | min us | max us | avg us (roofline pass) |",
            "|---|---|---|---|---|---|"]
    for r in stats:
        name = r["Name"]
        d = by_kernel.get(name, [])
        rp = d[W_ + K_: W_ + 2 * K_] if len(d) >= W_ + 2 * K_ else []
        rp_s = f"{sum(rp) / len(rp):.2f}" if rp else "-"
        text.append(f"| `{name[:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                    f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {rp_s} |")
    text += ["", "bench.py's own figures in the same run (HIP events on the launching stream):", "",
             f"- kernels_us: {res.get('kernels_us')}",
             f"- roofline ({dom}): achieved {res['roofline']['achieved']} {res['roofline']['unit']} = "
             f"{100 * res['roofline']['frac']:.1f}% of {res['roofline']['peak']}"]
    if res.get("roofline_extend"):
        re_ = res["roofline_extend"]
        text.append(f"- roofline_extend: {re_['achieved']} {re_['unit']} = {100 * re_['frac']:.1f}% of {re_['peak']}")
    text += [f"- ms_per_step {res['ms_per_step']} (cold median; p10/p90 {res['ms_per_step_spread']['p10']} / "
             f"{res['ms_per_step_spread']['p90']}), warm {res.get('ms_per_step_warm')}; "
             f"{res['value']} tokens/s", ""]
    path = os.path.join(ROOT, "profiles", f"{dom}_{wl}.md")
    with open(path, "w") as fh:
        fh.write("\n".join(text))
    print(path)


def measured_ceilings(stream, scratch):
    """What plain device work reaches on this GPU in the same run, beside the
    published peaks: a 1 GiB read (torch's max over the cold-flush buffer), a
    512 MiB device copy (bytes read + written) and an 8192^3 bf16 GEMM
    (torch.mm, the vendor BLAS); medians of 10 timed runs after 3 untimed."""
    import torch

    def med_ms(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
        for e0, e1 in ev:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))

    read_b = scratch.numel() * scratch.element_size()
    t_read = med_ms(lambda: scratch.max())
    src = torch.empty(1 << 29, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    t_copy = med_ms(lambda: dst.copy_(src))
    del src, dst
    n = 8192
    x = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    y = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    t_mm = med_ms(lambda: torch.mm(x, y))
    del x, y
    return {"hbm_read_gbps": round(read_b / (t_read * 1e-3) / 1e9, 1),
            "hbm_copy_gbps": round(2 * (1 << 29) / (t_copy * 1e-3) / 1e9, 1),
            "bf16_gemm_tflops": round(2 * n ** 3 / (t_mm * 1e-3) / 1e12, 1),
            "how": "1 GiB read (max), 512 MiB copy (read + written bytes), 8192^3 bf16 torch.mm; "
                   "medians of 10"}


def load_traffic(kernel, workload):
    """Measured HBM bytes per launch, or None when absent or taken on other sources."""
    path = traffic_record_path(kernel, workload)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        body = fh.read()
    try:
        rec = json.loads(body.split("```json", 1)[1].split("```", 1)[0])
    except (IndexError, ValueError):
        return None
    if rec.get("source_sha") != source_hash(kernel):
        return None
    return rec["hbm_bytes"]


def cascade_prefix(w, seq_lens, qsl, ext_min_rows=2, extend_on=True, hint=True):
    """Keys of the shared prefix that the library's cascade takes over from the
    split-K rows (0 when it does not apply), and whether the split-K launch
    computes the prefix rows' prefix part itself (prefix items, rather than
    the MFMA prefix pass): the same rules as the library's plan."""
    P = w.shared_prefix_blocks * w.block_size if hint else 0
    mfma_ok = w.kv_dtype in ("bf16", "fp8") and w.head_dim == 128 and w.io_dtype == "bf16"
    if P == 0 or not mfma_ok or os.environ.get("PA_DISABLE_CASCADE", "0") not in ("", "0"):
        return 0, False
    rows = 0
    for i in range(w.num_seqs):
        c, L = int(qsl[i + 1] - qsl[i]), int(seq_lens[i])
        if c == 0 or (extend_on and c >= ext_min_rows and mfma_ok):
            continue
        if L - c < P:
            return 0, False
        rows += c
    if not rows:
        return 0, False
    in_decode = rows * (w.num_q_heads // w.num_kv_heads) <= 1024 and \
        os.environ.get("PA_PREFIX_PASS", "0") in ("", "0")
    return P, in_decode


def multirow_chunk(w, c):
    """Whether the library runs a chunk of c rows as one multi-row split-K item
    (PA_MULTIROW=1: 2 <= c and c * g <= 32, bf16 and fp8 pools), as its plan does."""
    on = os.environ.get("PA_MULTIROW", "0") not in ("", "0")
    return on and w.kv_dtype != "f32" and c >= 2 and c * (w.num_q_heads // w.num_kv_heads) <= 32


def algorithmic_work(w, seq_lens, qsl, ext_min_rows=2, extend_on=True, prefix=0, fused=False,
                     prefix_in_decode=False, scatter_in_decode=False):
    """Bytes the split-K decode kernel must move, flops the extend kernel must
    do and flops of the shared-prefix attention, per step, by the per-unit
    formulas in the design notes.  With a shared prefix of `prefix` keys, the
    split-K rows' bytes count their own keys, and the prefix's K/V once per
    kv head when the split-K launch computes the prefix part itself
    (`prefix_in_decode`).  In the step with the KV update (`fused`), a
    decode row of a one-token request takes its newest key from the input
    rows and also writes them to the pool; when the split-K launch also
    carries the scatter of the prefill chunks' rows (`scatter_in_decode`),
    their input rows read and pool rows written count as its bytes too (a
    chunk of at most 128 (row, head) columns per kv head writes its own rows
    in the extend kernel).  A multi-row split-K item reads its request's K/V
    once for all of its rows (and, in the step with the KV update, writes the
    rows' new K/V first)."""
    b_kv, b_io = ELEM[w.kv_dtype], ELEM[w.io_dtype]
    H, Hq, D, S = w.num_kv_heads, w.num_q_heads, w.head_dim, w.block_size
    dec_bytes = 0
    ext_flops = 0
    ext_bytes = 0
    pre_flops = 0
    for i in range(w.num_seqs):
        c, L = int(qsl[i + 1] - qsl[i]), int(seq_lens[i])
        if c == 0:
            continue
        use_ext = (extend_on and c >= ext_min_rows and w.kv_dtype in ("bf16", "fp8") and D == 128
                   and not multirow_chunk(w, c))
        if multirow_chunk(w, c):
            dec_bytes += (L - prefix) * H * D * 2 * b_kv + c * Hq * D * b_io + (-(-L // S) - prefix // S) * 4
            if fused:
                dec_bytes += c * H * D * 2 * (b_io + b_kv)
            pre_flops += 4 * Hq * D * prefix * c
        elif use_ext:
            ext_flops += 4 * Hq * D * sum(L - c + t + 1 for t in range(c))
            ext_bytes += L * H * D * 2 * b_kv + c * Hq * D * 2 * b_io
            if scatter_in_decode and c * (Hq // H) > 128:
                dec_bytes += c * H * D * 2 * (b_io + b_kv)
        else:
            for t in range(c):
                Lv = L - c + t + 1
                dec_bytes += (Lv - prefix) * H * D * 2 * b_kv + Hq * D * b_io + (-(-Lv // S) - prefix // S) * 4
                if fused and c == 1:
                    dec_bytes += H * D * 2 * (b_io - b_kv) + H * D * 2 * b_kv
                pre_flops += 4 * Hq * D * prefix
    if prefix_in_decode:
        dec_bytes += prefix * H * D * 2 * b_kv
    return dec_bytes, ext_flops, ext_bytes, pre_flops


def table_walk_kv_bytes(w, seq_lens, qsl, ext_min_rows=2, extend_on=True):
    """K+V bytes of every split-K row's whole visible key range, each row
    walking its own block table (a shared prefix counts once per row): the
    per-request work that the shared-prefix pass takes over."""
    b_kv, H, D = ELEM[w.kv_dtype], w.num_kv_heads, w.head_dim
    total = 0
    for i in range(w.num_seqs):
        c, L = int(qsl[i + 1] - qsl[i]), int(seq_lens[i])
        if c == 0 or (extend_on and c >= ext_min_rows and w.kv_dtype in ("bf16", "fp8") and D == 128):
            continue
        total += sum(L - c + t + 1 for t in range(c)) * H * D * 2 * b_kv
    return total


def unique_kv_bytes(w, seq_lens, qsl, prefix=0, ext_min_rows=2, extend_on=True):
    """K+V bytes of the distinct pool slots the split-K rows read (a block
    shared by several requests counts once; keys before `prefix` are the
    cascade pass's): what HBM must deliver at least once."""
    b_kv = ELEM[w.kv_dtype]
    S = w.block_size
    seen = {}
    for i in range(w.num_seqs):
        c, L = int(qsl[i + 1] - qsl[i]), int(seq_lens[i])
        if c == 0 or (extend_on and c >= ext_min_rows and w.kv_dtype in ("bf16", "fp8") and w.head_dim == 128):
            continue
        for b in range(prefix // S, -(-L // S)):
            blk = int(w.block_table[i, b])
            seen[blk] = max(seen.get(blk, 0), min(S, L - b * S))
    return sum(seen.values()) * w.num_kv_heads * w.head_dim * 2 * b_kv


def main():
    a = parse()
    if a.traffic_ingest:
        traffic_ingest(a)
        return
    if a.counters_ingest:
        counters_ingest(a)
        return
    if a.trace_summary:
        trace_summary(a)
        return
    if a.gpus != 1:
        print(json.dumps({"error": "the step runs on one GPU only (no multi-GPU path); --gpus must be 1",
                          "n_gpus": a.gpus}), flush=True)
        sys.exit(2)

    import torch

    from paged_kv_cache_pool_amd import binding as B
    from paged_kv_cache_pool_amd import runner
    from paged_kv_cache_pool_amd import workloads as W

    if a.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n}), flush=True)
        return

    t0 = time.time()
    w = W.make(a.config, a.seed)
    print(f"[bench] workload {w.name}: generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()
    step = runner.GpuStep(w, stream=stream, fused=not a.separate)
    print(f"[bench] device set-up done ({time.time() - t0:.1f}s)", file=sys.stderr, flush=True)

    for _ in range(a.warmup):
        step.run()
    torch.cuda.synchronize()

    # A 1 GiB read before a cold step evicts L2 and the 256 MB Infinity Cache
    # (clean lines: no write-back is left for the step to pay); it runs before
    # the step's first event, so only the step is between its events.
    scratch = torch.ones(1 << 27, dtype=torch.int64, device="cuda")

    def cold_steps(n):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for e0, e1 in evs:
            scratch.max()
            e0.record(stream)
            step.run()
            e1.record(stream)
        return evs

    # timed region: K cold steps, bracketed by synchronisations
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    evs = cold_steps(a.steps)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    per_step = np.array([e0.elapsed_time(e1) for e0, e1 in evs])
    ms_per_step = float(np.median(per_step))
    spread = {"p10": round(float(np.percentile(per_step, 10)), 5),
              "p50": round(ms_per_step, 5),
              "p90": round(float(np.percentile(per_step, 90)), 5)}

    # K more cold steps with HIP events around every kernel launch on the
    # stream it runs on (the library records them): the kernels' durations
    B.profile_enable(True)
    cold_steps(a.steps)
    torch.cuda.synchronize()
    kernels = {}
    for name in ("k_slot_mapping", "k_write_kv", "k_write_new", "k_prefix", "k_decode", "k_merge",
                 "k_extend"):
        n, ms = B.profile_read(name)
        if n:
            kernels[name] = {"launches": n, "avg_us": 1000.0 * ms / n}
    B.profile_enable(False)

    # the same K steps back to back with warm caches (inputs of the previous
    # identical step partly cached), beside the cold figure
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(a.steps):
        step.run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_warm = e0.elapsed_time(e1) / a.steps
    # the other form of the step on the same pool and inputs (the KV write is
    # idempotent), for comparison (cold steps, median)
    other = None
    if a.compare:
        step.fused = a.separate
        for _ in range(a.warmup):
            step.run()
        torch.cuda.synchronize()
        evo = cold_steps(a.steps)
        torch.cuda.synchronize()
        other = round(float(np.median([x0.elapsed_time(x1) for x0, x1 in evo])), 5)
        step.fused = not a.separate

    graph_ms = None
    graph_layers = None
    if a.graph:
        # the step captured on a side stream, then replayed on the step's
        # stream: warm back-to-back replays, against the warm eager figure
        gs = torch.cuda.Stream()
        gs.wait_stream(stream)
        step.stream = gs
        with torch.cuda.stream(gs):
            step.run()
        gs.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=gs):
            step.run()
        step.stream = stream
        torch.cuda.synchronize()
        for _ in range(a.warmup):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(a.steps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        graph_ms = round(e0.elapsed_time(e1) / a.steps, 5)
        del g
        # the attention layers of one model step: --graph-layers steps, each on
        # its own pool and inputs, launched eagerly back to back against one
        # graph holding all of them (launch gaps between layers are paid once
        # per graph), warm, per layer
        nl = max(1, a.graph_layers)
        layers = [step] + [runner.GpuStep(w, stream=stream, fused=step.fused) for _ in range(nl - 1)]
        for _ in range(a.warmup):
            for ly in layers:
                ly.run()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(a.steps):
            for ly in layers:
                ly.run()
        e1.record(stream)
        torch.cuda.synchronize()
        eager_layer = e0.elapsed_time(e1) / (a.steps * nl)
        gs.wait_stream(stream)
        for ly in layers:
            ly.stream = gs
        with torch.cuda.stream(gs):
            for ly in layers:
                ly.run()
        gs.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=gs):
            for ly in layers:
                ly.run()
        for ly in layers:
            ly.stream = stream
        torch.cuda.synchronize()
        for _ in range(a.warmup):
            g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(a.steps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        graph_layers = {"layers": nl, "eager_ms_per_layer_warm": round(eager_layer, 5),
                        "replay_ms_per_layer_warm": round(e0.elapsed_time(e1) / (a.steps * nl), 5)}
        del g, layers
    ceilings = measured_ceilings(stream, scratch)
    del scratch

    T = w.num_tokens
    tokens_per_s = T / (ms_per_step / 1000.0)
    qsl, sl = B.prepare_metadata(w.num_computed, w.num_scheduled)
    ext_on = os.environ.get("PA_DISABLE_EXTEND", "0") in ("", "0")
    ext_min = int(os.environ.get("PA_EXTEND_MIN_ROWS", "2"))
    prefix, prefix_in_decode = cascade_prefix(w, sl, qsl, ext_min, ext_on,
                                              hint=step.batch.num_common_prefix_blocks > 0)
    # the scatter of the chunks' rows rides in the split-K launch when no
    # launch of its own ran (one-call step with split-K rows)
    scatter_in_decode = (not a.separate and "k_decode" in kernels and "k_write_new" not in kernels
                         and "k_extend" in kernels)
    dec_bytes, ext_flops, ext_bytes, pre_flops = algorithmic_work(
        w, sl, qsl, ext_min, ext_on and "k_extend" in kernels, prefix, fused=not a.separate,
        prefix_in_decode=prefix_in_decode, scatter_in_decode=scatter_in_decode)

    # dominant kernel: the attention kernel that takes the longer time.  The
    # extend kernel is priced against MFMA when its work is compute-heavy
    # (prefill chunks), against HBM when it is not (short verify chunks over
    # long histories: flops per byte below the peaks' ratio)
    t_dec = kernels.get("k_decode", {}).get("avg_us", 0.0) if dec_bytes > 0 else 0.0
    t_ext = kernels.get("k_extend", {}).get("avg_us", 0.0) if ext_flops > 0 else 0.0
    ext_hbm = ext_flops > 0 and ext_flops / max(ext_bytes, 1) < MFMA_BF16_PEAK_TFLOPS / HBM_PEAK_GBPS * 1e3
    if t_ext > t_dec and ext_hbm:
        dom = "k_extend"
        achieved = ext_bytes / (t_ext * 1e-6) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": load_traffic(dom, w.name), "algorithmic_bytes_per_launch": ext_bytes}
    elif t_dec >= t_ext:
        dom = "k_decode"
        achieved = dec_bytes / (kernels[dom]["avg_us"] * 1e-6) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": load_traffic(dom, w.name), "algorithmic_bytes_per_launch": dec_bytes}
    else:
        dom = "k_extend"
        achieved = ext_flops / (kernels[dom]["avg_us"] * 1e-6) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1),
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": load_traffic(dom, w.name),
                "algorithmic_flops_per_launch": ext_flops}

    # the extend kernel against the bf16 MFMA peak whenever the step has
    # prefill rows (its flops: visible (query, key) pairs only)
    roof_ext = None
    if ext_flops and "k_extend" in kernels:
        achieved = ext_flops / (kernels["k_extend"]["avg_us"] * 1e-6) / 1e12
        roof_ext = {"kernel": "k_extend", "bound": "mfma", "achieved": round(achieved, 1),
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                    "traffic": load_traffic("k_extend", w.name),
                    "algorithmic_flops_per_launch": ext_flops}

    # the same achieved figures against what plain device work reaches here
    for r in (roof, roof_ext):
        if r is None:
            continue
        ceil = ceilings["hbm_read_gbps"] if r["bound"] == "hbm" else ceilings["bf16_gemm_tflops"]
        r["frac_of_measured"] = round(r["achieved"] / ceil, 4)

    cpu = None
    if a.cpu_seconds > 0:
        import oracle as O
        pool = O.build_pool(w)
        # a step of more than 2048 rows is sampled: the attention of every
        # k-th row (slots and write of all rows), scaled to tokens/s by rows
        rows = None if T <= 2048 else np.arange(0, T, -(-T // 512), dtype=np.int32)
        n_rows = T if rows is None else len(rows)
        reps, t_cpu = 0, 0.0
        while t_cpu < a.cpu_seconds and reps < 1000:
            t1 = time.perf_counter()
            O.run_step(w, pool=pool, tokens=rows)
            t_cpu += time.perf_counter() - t1
            reps += 1
        what = (f"whole step of this workload ({T} tokens: slots, write, attention)" if rows is None else
                f"slots and write of all {T} tokens, attention of {n_rows} rows (every "
                f"{int(rows[1] - rows[0])}th)")
        cpu = {"value": round(n_rows * reps / t_cpu, 2), "unit": "tokens/s", "cores": O.num_threads(),
               "kind": "oracle", "sample": f"{what}, {reps} repetition(s), {t_cpu:.1f}s, fp64"}

    # dispatch placement the planners rely on (diagnostic, after the timed
    # region): a fraction below 1 costs speed, never exactness
    try:
        placement = B.placement_check()
    except B.PaError as e:
        placement = {"error": str(e)}

    out = {
        "metric": "tokens/s per paged-attn step + decode KV GB/s (% of HBM peak), 1 MI355X",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.kv_dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "tokens_per_step": T,
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "block_size": w.block_size, "kv_dtype": w.kv_dtype,
                   "num_blocks": w.num_blocks, "context_total": int(sl.sum()),
                   "context_min": int(sl.min()), "context_max": int(sl.max()), "seed": a.seed},
        "roofline": roof,
        **({"roofline_extend": roof_ext} if roof_ext is not None and dom != "k_extend" else {}),
        "cpu_baseline": cpu,
        "timing": "cold caches: a 1 GiB read before each step, outside its events; median of the "
                  "steps' HIP-event times",
        "ms_per_step_spread": spread,
        "ms_per_step_warm": round(ms_warm, 5),
        "timed_region_wall_s": round(t_wall, 4),
        "kernels_us": {k: round(v["avg_us"], 2) for k, v in kernels.items()},
        "step_form": "separate calls" if a.separate else "one call with the KV update",
        **({("ms_per_step_one_call" if a.separate else "ms_per_step_separate_calls"): other}
           if other is not None else {}),
        **({"ms_per_step_graph_replay_warm": graph_ms} if graph_ms is not None else {}),
        **({"graph_layers": graph_layers} if graph_layers is not None else {}),
        "decode_kv_gbps": roof["achieved"] if dom == "k_decode" else None,
        "placement": placement,
        "measured_ceilings": ceilings,
    }
    if dom == "k_decode":
        # pool K/V bytes by two counts beside the algorithmic ones: every row
        # walking its own block table (logical), and the distinct slots read
        # (unique); they differ where requests share blocks
        t_us = kernels["k_decode"]["avg_us"]
        logical = table_walk_kv_bytes(w, sl, qsl, ext_min, ext_on and "k_extend" in kernels)
        uniq = unique_kv_bytes(w, sl, qsl, 0 if prefix_in_decode else prefix, ext_min,
                               ext_on and "k_extend" in kernels)
        out["decode_kv_bytes_algorithmic"] = dec_bytes
        out["decode_kv_bytes_logical"] = logical
        out["decode_kv_gbps_logical"] = round(logical / (t_us * 1e-6) / 1e9, 1)
        out["decode_kv_bytes_unique"] = uniq
        out["decode_kv_gbps_unique"] = round(uniq / (t_us * 1e-6) / 1e9, 1)
    if prefix:
        out["prefix_keys"] = prefix
        out["prefix_attention"] = "split-K prefix items" if prefix_in_decode else "MFMA prefix pass"
    if pre_flops and "k_prefix" in kernels:
        out["prefix_tflops"] = round(pre_flops / (kernels["k_prefix"]["avg_us"] * 1e-6) / 1e12, 1)
    if ext_flops:
        out["extend_tflops"] = round(ext_flops / (kernels["k_extend"]["avg_us"] * 1e-6) / 1e12, 1) \
            if "k_extend" in kernels else None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
