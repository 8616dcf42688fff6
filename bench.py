"""Benchmark of the sliding-window attention backward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload c3|c3_atomic|c1|c2_4k|c2_8k|c2_4k_det|c2_8k_det|c4|c4_f16|c5]
    python bench.py --copy-calibration ...      (appends a copy of known size)
    python bench.py --summarize-stats DIR --out FILE --command CMD
    python bench.py --summarize-traffic FETCH_DIR WRITE_DIR --out FILE --command CMD
    python bench.py --summarize-counters PMC_DIR... --out FILE --command CMD... --workload W

A step is one full backward, sdpa_bwd_run: the dot preprocess, the main
window-bounded kernel with its dQ accumulation (ordered relay, fp32 atomics
at the streaming kernel's chunk boundaries, or the separate q-major dQ
pass), the dQ conversion where an accumulator is used, and dSink (with
sinks), on inputs already resident in HBM.  The default workload is the
long-sequence shape of the pages' measurements: batch 2, 16 heads,
head_dim 64, S = 32768, causal top-left with a left window of 128, bf16,
deterministic relay.  Prints one JSON line; ``extra`` carries the other
workloads and the forward's time per call for each.

FLOPs count attended (query, key) pairs only: 10 * head_dim per pair per
query head for the backward, 4 * head_dim for the forward.  The roofline
entry is for the dominant kernel (the streaming main kernel at the default
workload), timed with HIP events recorded on its launch stream around every
launch of a second run of as many steps (the timed steps themselves run
uninstrumented, since the event packets lengthen a step).  Its ``traffic`` is the HBM bytes per launch that rocprofv3's
FETCH_SIZE and WRITE_SIZE counters read for it, each divided by what the
same counter reads per byte for an elementwise copy of known size; the
figures are kept in a text summary under profiles/ together with a hash of
the kernel's sources, and ``traffic`` is null when the sources no longer
match.
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
METRIC = "SWA backward ms & TFLOP/s (attended pairs), b2 h16 d64 W128 S=4k/8k/32k"

# the dominant kernel of the default workload and the files that define it
MAIN_KERNEL = "bwd_stream_kernel"
MAIN_KERNEL_SOURCES = [
    "sliding_window_attention_flash_amd/csrc/bwd_stream.hip",
    "sliding_window_attention_flash_amd/csrc/common.h",
    "sliding_window_attention_flash_amd/csrc/kernels.h",
    "sliding_window_attention_flash_amd/csrc/swa_sched.h",
    "sliding_window_attention_flash_amd/build.py",
]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bwd_stream_c3_s32768_hbm_traffic.txt")
COPY_BYTES = 1 << 30  # calibration copy: reads and writes this many bytes
COPY_KERNEL = "neg_kernel"


def _hip():
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    return lib


def workloads():
    from sliding_window_attention_flash_amd.synth import CONFIGS
    c3 = CONFIGS["c3"]
    return {
        "c3": c3,
        "c3_atomic": c3.with_(name=c3.name.replace("_det", "_atomic"), deterministic=False),
        "c1": CONFIGS["c1"],
        "c2_4k": CONFIGS["c2_4k"],
        "c2_8k": CONFIGS["c2_8k"],
        "c2_4k_det": CONFIGS["c2_4k"].with_(name=CONFIGS["c2_4k"].name + "_det", deterministic=True),
        "c2_8k_det": CONFIGS["c2_8k"].with_(name=CONFIGS["c2_8k"].name + "_det", deterministic=True),
        "c4": CONFIGS["c4"],
        "c4_f16": CONFIGS["c4_f16"],
        "c5": CONFIGS["c5"],
    }


def main_kernel_bytes(w) -> int:
    """Algorithmic HBM bytes of one bwd_main launch: Q, dO read and dQ
    written once per query-head row, plus the row's LSE and delta (fp32);
    K, V read and dK, dV written once per kv-head row."""
    from sliding_window_attention_flash_amd.synth import Workload  # noqa: F401
    rows_q = sum(w.valid_len_q()) * w.heads_q
    rows_kv = sum(w.valid_len_kv()) * w.heads_kv
    return rows_q * (3 * w.head_dim * 2 + 8) + rows_kv * (4 * w.head_dim * 2)


def time_backward(w, steps, warmup, seed=0, forward=False):
    """Per-step wall time of the backward (ms), the average of the main
    kernel's HIP-event times (ms), the relay expiries, and with forward=True
    also the forward's wall time per call (ms)."""
    import torch
    from sliding_window_attention_flash_amd import api
    from sliding_window_attention_flash_amd.synth import make_inputs

    inp = make_inputs(w, device="cuda", seed=seed)
    mk = dict(causal=w.causal, bottom_right=w.bottom_right, window_left=w.window_left,
              window_right=w.window_right, scale=w.softmax_scale, cu_seqlens_q=inp["cu_seqlens_q"],
              cu_seqlens_kv=inp["cu_seqlens_kv"],
              seq_lens_q=inp["seq_lens_q"], seq_lens_kv=inp["seq_lens_kv"])
    if w.layout == "thd":
        mk.update(max_seqlen_q=w.seq_q, max_seqlen_kv=w.seq_kv)
    fw = api.Forward(inp["q"], inp["k"], inp["v"], sink=inp["sink"], **mk)
    o, lse = fw.run()
    bw = api.Backward(inp["q"], inp["k"], inp["v"], o, inp["dO"], lse, deterministic=w.deterministic,
                      sink=inp["sink"], **mk)
    hip = _hip()
    ev = []
    for _ in range(2 * steps):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        ev.append(e)
    for _ in range(warmup):
        bw.run()
    # the timed steps, uninstrumented
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        bw.run()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    # the same number of steps again, with HIP events recorded on the launch
    # stream around the main kernel of each (the events add stream packets,
    # so these steps are not the timed ones)
    for s in range(steps):
        bw.run_events(ev[2 * s].value, ev[2 * s + 1].value)
    torch.cuda.synchronize()
    main_ms = []
    for s in range(steps):
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), ev[2 * s], ev[2 * s + 1]) == 0
        main_ms.append(ms.value)
    for e in ev:
        hip.hipEventDestroy(e)
    expiries = bw.relay_expiries() if w.deterministic else 0
    if not forward:
        return wall * 1e3, sum(main_ms) / len(main_ms), expiries
    for _ in range(max(3, warmup // 5)):
        fw.run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fw.run()
    torch.cuda.synchronize()
    fwd_ms = (time.perf_counter() - t0) / steps * 1e3
    return wall * 1e3, sum(main_ms) / len(main_ms), expiries, fwd_ms


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in MAIN_KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read() + b"\0")
    return h.hexdigest()


def stored_traffic(w):
    """HBM bytes per launch of the main kernel from the committed counter
    summary, or None if there is none for this workload or the kernel's
    sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = [json.loads(x[len("TRAFFIC "):]) for x in fh if x.startswith("TRAFFIC ")]
    except OSError:
        return None
    for r in rec:
        if r.get("workload") == w.name and r.get("source_sha256") == kernel_source_hash():
            return r["traffic_bytes_per_launch"]
    return None


def copy_calibration():
    """An elementwise kernel that reads COPY_BYTES and writes COPY_BYTES
    (torch.neg into a second buffer), launched three times."""
    import torch
    x = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    x.zero_()
    y = torch.empty_like(x)
    for _ in range(3):
        torch.neg(x, out=y)
    torch.cuda.synchronize()


# ---- profile summaries --------------------------------------------------------


def _rows(path):
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def _find(d, suffix):
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(root, f)
    raise FileNotFoundError(f"no *{suffix} under {d}")


def _timed_launch_avg_us(d, steps):
    """Average duration (us) of the main kernel over its last ``steps``
    dispatches in the kernel trace (the event-timed ones, which follow the
    warm-up and the uninstrumented timed steps)."""
    rows = [r for r in _rows(_find(d, "kernel_trace.csv")) if MAIN_KERNEL in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    last = rows[-steps:]
    return sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in last) / len(last) / 1e3, len(last)


def summarize_stats(d, out, command, bench_json=None, steps=None, workload="c3"):
    rows = _rows(_find(d, "kernel_stats.csv"))
    lines = [f"# rocprofv3 kernel statistics, workload {workloads()[workload].name}", "", "command:",
             f"    {command}", "",
             f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}  kernel"]
    for r in rows:
        name = r["Name"]
        short = name if len(name) < 90 else name[:87] + "..."
        lines.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} {float(r['MinNs']) / 1e3:10.2f} "
                     f"{float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):6.2f}  {short}")
    if bench_json:
        with open(bench_json) as fh:
            b = json.loads([x for x in fh if x.startswith("{")][-1])
        lines += ["", "bench line of the same run (HIP events on the launch stream, profiler attached):",
                  f"    main_kernel_ms = {b['extra']['main_kernel_ms']:.4f}, ms_per_step = {b['ms_per_step']:.4f}"]
    if steps and any(MAIN_KERNEL in r["Name"] for r in rows):
        avg, n = _timed_launch_avg_us(d, steps)
        lines += ["", f"{MAIN_KERNEL} over the event-timed launches (last {n} dispatches of the kernel trace): "
                      f"avg {avg:.2f} us"]
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter_means(d, counter):
    """{kernel name: (dispatches, mean counter value per dispatch)}"""
    acc = {}
    for r in _rows(_find(d, "counter_collection.csv")):
        if r["Counter_Name"] != counter:
            continue
        k = r["Kernel_Name"]
        n, v = acc.get(k, (0, 0.0))
        acc[k] = (n + 1, v + float(r["Counter_Value"]))
    return {k: (n, v / n) for k, (n, v) in acc.items()}


def _pick(means, pat):
    hits = [(k, nv) for k, nv in means.items() if pat in k]
    if len(hits) != 1:
        raise RuntimeError(f"expected one kernel matching {pat!r}, found {[k[:80] for k, _ in hits]}")
    return hits[0][1]


def summarize_traffic(fetch_dir, write_dir, out, command, workload):
    w = workloads()[workload]
    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")
    nf, kf = _pick(fetch, MAIN_KERNEL)
    nw, kw = _pick(write, MAIN_KERNEL)
    _, cf = _pick(fetch, COPY_KERNEL)
    _, cw = _pick(write, COPY_KERNEL)
    copy_kib = COPY_BYTES / 1024
    ff, fw = cf / copy_kib, cw / copy_kib  # counter KiB per byte-KiB moved
    traffic = kf * 1024 / ff + kw * 1024 / fw
    algo = main_kernel_bytes(w)
    rec = {"kernel": MAIN_KERNEL, "workload": w.name, "launches_fetch": nf, "launches_write": nw,
           "fetch_kib_per_launch": kf, "write_kib_per_launch": kw, "copy_bytes": COPY_BYTES,
           "copy_fetch_kib": cf, "copy_write_kib": cw, "fetch_factor": ff, "write_factor": fw,
           "traffic_bytes_per_launch": traffic, "algorithmic_bytes_per_launch": algo,
           "source_sha256": kernel_source_hash()}
    lines = [f"# HBM traffic of {MAIN_KERNEL}, workload {w.name}", "",
             "commands (FETCH_SIZE pass, then WRITE_SIZE pass):", *[f"    {c}" for c in command], "",
             f"FETCH_SIZE per launch   {kf:14.1f} KiB  ({nf} launches)",
             f"WRITE_SIZE per launch   {kw:14.1f} KiB  ({nw} launches)",
             f"calibration copy of {COPY_BYTES} bytes ({COPY_KERNEL}): FETCH_SIZE {cf:.1f} KiB, "
             f"WRITE_SIZE {cw:.1f} KiB",
             f"factors (counter bytes per byte moved): fetch {ff:.4f}, write {fw:.4f}",
             f"HBM traffic per launch  {traffic / 1e6:14.2f} MB  (fetch {kf * 1024 / ff / 1e6:.2f} MB, "
             f"write {kw * 1024 / fw / 1e6:.2f} MB)",
             f"algorithmic bytes       {algo / 1e6:14.2f} MB  (traffic / algorithmic = {traffic / algo:.3f})",
             "", "TRAFFIC " + json.dumps(rec)]
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


SQ_KERNELS = ("bwd_stream_kernel", "bwd_main_kernel", "bwd_dq_kernel", "bwd_dot_kernel", "bwd_dsink_kernel",
              "fwd_kernel")
CLOCK_GHZ = 2.4   # MI355X peak engine clock
N_SIMD = 256 * 4  # compute units x SIMDs


def summarize_counters(dirs, out, commands, workload):
    """Per-kernel averages (per dispatch) of SQ counters from rocprofv3 --pmc
    runs, with instructions per wave and the MFMA-busy fraction of the
    kernel's SIMD cycles (SQ_VALU_MFMA_BUSY_CYCLES, summed over SIMDs, over
    dispatch duration x 2.4 GHz x 1024 SIMDs)."""
    import collections
    vals = collections.defaultdict(lambda: collections.defaultdict(dict))
    dur = collections.defaultdict(dict)
    for d in dirs:
        for r in _rows(_find(d, "counter_collection.csv")):
            k = next((n for n in SQ_KERNELS if n in r["Kernel_Name"]), None)
            if k is None:
                continue
            key = (d, r["Dispatch_Id"])
            vals[k][r["Counter_Name"]][key] = vals[k][r["Counter_Name"]].get(key, 0.0) + float(r["Counter_Value"])
            dur[k][key] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    lines = [f"# SQ counters per kernel, workload {workloads()[workload].name}", "",
             "commands (one rocprofv3 --pmc pass each):"] + [f"    {c}" for c in commands] + [""]
    for k in SQ_KERNELS:
        if k not in vals:
            continue
        avg = {c: sum(v.values()) / len(v) for c, v in vals[k].items()}
        d_ns = sum(dur[k].values()) / len(dur[k])
        lines.append(f"{k}: {len(dur[k])} dispatches, {d_ns / 1e3:.1f} us per dispatch under the counters")
        for c in sorted(avg):
            lines.append(f"    {c:28s} {avg[c]:14.4g}")
        waves = avg.get("SQ_WAVES")
        if waves:
            per = {c[len('SQ_INSTS_'):]: avg[c] / waves for c in avg if c.startswith("SQ_INSTS_")}
            lines.append("    instructions per wave      " + ", ".join(f"{c} {v:.0f}" for c, v in sorted(per.items())))
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
            frac = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (d_ns * CLOCK_GHZ * N_SIMD)
            lines.append(f"    MFMA busy / SIMD cycles    {frac:.3f}")
        lines.append("")
    with open(out, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def cpu_baseline(w):
    """The fp64 oracle's backward timed on the whole workload when it is a
    dense multi-head one (the oracle runs one (sequence, kv head) unit per
    host thread), scaled to attended TFLOP/s; other workloads are sampled to
    one sequence."""
    import oracle
    from sliding_window_attention_flash_amd.synth import make_inputs

    ws = w if w.layout == "bhsd" and w.batch * w.heads_kv <= 64 else w.with_(batch=1, name=w.name + "_b0")
    inp = make_inputs(ws, device="cpu", seed=0)
    p = oracle.Problem.dense(ws.batch, ws.heads_q, ws.heads_kv, ws.seq_q, ws.seq_kv, ws.head_dim,
                             causal=ws.causal, bottom_right=ws.bottom_right,
                             window_left=ws.window_left, scale=ws.softmax_scale)
    t0 = time.perf_counter()
    oracle.backward(p, inp["q"], inp["k"], inp["v"], inp["dO"], None)
    dt = time.perf_counter() - t0
    pairs = oracle.attended_pairs(p) * ws.heads_q
    flops = 10.0 * ws.head_dim * pairs
    units = ws.batch * ws.heads_kv
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": min(oracle.num_threads(), units),
            "kind": "oracle",
            "sample": f"fp64 oracle backward (forward recompute included) on {ws.batch} sequence(s) x "
                      f"{ws.heads_q} head(s) of {w.name}: {pairs} attended pairs in {dt:.2f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="c3", choices=sorted(workloads()))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the 4k / 8k / atomic side timings")
    ap.add_argument("--copy-calibration", action="store_true",
                    help=f"after timing, copy {COPY_BYTES} bytes three times (counter calibration)")
    ap.add_argument("--summarize-stats", metavar="DIR")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-counters", nargs="+", metavar="PMC_DIR")
    ap.add_argument("--bench-json")
    ap.add_argument("--out")
    ap.add_argument("--command", action="append", default=[])
    args = ap.parse_args()
    if args.summarize_stats:
        summarize_stats(args.summarize_stats, args.out, " ".join(args.command), args.bench_json, args.steps,
                        args.workload)
        return
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, args.out, args.command, args.workload)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.out, args.command, args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the timed kernel is "
              "one GPU's share of the work at its full shape", file=sys.stderr)
        sys.exit(2)

    import torch
    from sliding_window_attention_flash_amd.synth import flops

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    wl = workloads()
    w = wl[args.workload]
    ms, main_ms, exp, fwd_ms = time_backward(w, args.steps, args.warmup, forward=True)
    fl = flops(w)
    tflops = fl / (ms * 1e-3) / 1e12
    nbytes = main_kernel_bytes(w)
    achieved = nbytes / (main_ms * 1e-3) / 1e9
    extra = {"main_kernel": MAIN_KERNEL, "main_kernel_ms": main_ms,
             "main_kernel_algorithmic_bytes": nbytes,
             "main_kernel_attended_tflops": fl / (main_ms * 1e-3) / 1e12,
             "frac_bf16_mfma_peak": tflops / BF16_MFMA_PEAK_TFLOPS, "relay_expiries": exp,
             "attended_flops": fl, "forward_ms": fwd_ms,
             "forward_tflops": 0.4 * fl / (fwd_ms * 1e-3) / 1e12}
    if not args.no_extra:
        # every other workload, timed the same way (the large GQA one with
        # fewer steps); each entry names its workload's shape
        for name in ("c3_atomic", "c1", "c2_4k", "c2_8k", "c2_4k_det", "c2_8k_det", "c4", "c4_f16", "c5"):
            if name == args.workload:
                continue
            wx = wl[name]
            big = wx.batch * wx.heads_q * wx.seq_q * wx.head_dim > (1 << 30)
            st, wu = (max(3, args.steps // 4), max(3, args.warmup // 10)) if big else (max(5, args.steps // 2), args.warmup)
            m2, mm2, _, fm2 = time_backward(wx, st, wu, forward=True)
            extra[name] = {"workload": wx.name, "ms": m2, "tflops": flops(wx) / (m2 * 1e-3) / 1e12, "main_ms": mm2,
                           "frac_bf16_mfma_peak": flops(wx) / (m2 * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                           "forward_ms": fm2, "forward_tflops": 0.4 * flops(wx) / (fm2 * 1e-3) / 1e12}
    line = {
        "metric": METRIC, "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads_q": w.heads_q, "heads_kv": w.heads_kv,
                   "head_dim": w.head_dim, "seq_len": w.seq_q, "window_left": w.window_left,
                   "mask": "causal_bottom_right" if w.bottom_right else "causal_top_left",
                   "dq_mode": "relay" if w.deterministic else "atomic"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": stored_traffic(w)},
        "extra": extra,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)
    if args.copy_calibration:
        copy_calibration()


if __name__ == "__main__":
    main()
