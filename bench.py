"""Benchmark of the sliding-window attention backward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--repeats R]
    python bench.py --copy-calibration ...      (appends a copy of known size)
    python bench.py --summarize-stats DIR --out FILE --command CMD
    python bench.py --summarize-traffic FETCH_DIR WRITE_DIR --out FILE --command CMD
    python bench.py --summarize-counters PMC_DIR... --out FILE --command CMD... --workload W

A step is one full backward, sdpa_bwd_run: the dot preprocess, the main
window-bounded kernel with its dQ accumulation (ordered relay, fp32 atomics
at the streaming kernel's chunk boundaries, or the separate q-major dQ
pass), and dSink (with sinks), on inputs already resident in HBM.  The
default workload is the long-sequence shape of the pages' measurements:
batch 2, 16 heads, head_dim 64, S = 32768, causal top-left with a left
window of 128, bf16, deterministic relay.  Prints one JSON line; ``extra``
carries every other workload.

Timing follows the pages' protocol (cudnn-frontend PR #2352, Measurement:
three repeats with fresh tensors, median per repeat, warm caches): each
repeat draws fresh inputs, runs the forward, then W warm-up steps and K
timed steps with a HIP event recorded on the launch stream between
consecutive steps; a repeat's figure is the median of its K per-step times,
and the reported step time is the median over the repeats.  Before the first
repeat of each workload the backward also runs for at least 0.5 s of wall
time, whatever W is, so that the first timed step does not meet an idle,
clocked-down GPU.  The K steps of each repeat are also timed as a whole with
host clocks (``host_mean_ms``), which shows what the per-step events cost.

FLOPs count attended (query, key) pairs only: 10 * head_dim per pair per
query head for the backward, 4 * head_dim for the forward.  Each workload
reports the fraction of bf16 MFMA peak and the fraction of its attainable
roofline, min(MFMA peak, arithmetic intensity x 8 TB/s), with the
compulsory bytes of Q, O, dO, dQ (per query-head row), K, V, dK, dV (per
kv-head row) and LSE.  The roofline entry of the JSON line is for the
dominant kernel (the streaming main kernel at the default workload), timed
with HIP events around every launch of a separate run; its ``traffic`` is
the HBM bytes per launch that rocprofv3's FETCH_SIZE and WRITE_SIZE
counters read for it, each divided by what the same counter reads per byte
for an elementwise copy of known size; the figures are kept in a text
summary under profiles/ together with a hash of the kernel's sources, and
``traffic`` is null when the sources no longer match.

The CPU leg (skipped with --no-cpu-baseline) runs the fp64 oracle on the
same inputs as each workload's last repeat: its wall time on the host's
cores, and the per-gradient parity errors of the GPU outputs (relative
Frobenius error and max-abs error over max|ref|), on the whole workload or,
where that is too slow, on whole batch entries or sequences (named in
``sample``).
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
    lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    return lib


def workloads():
    from sliding_window_attention_flash_amd.synth import CONFIGS
    c3 = CONFIGS["c3"]
    return {
        "c3": c3,
        "c3_atomic": c3.with_(name=c3.name.replace("_det", "_atomic"), deterministic=False, engine=1),
        "c1": CONFIGS["c1"],
        "c2_4k": CONFIGS["c2_4k"],
        "c2_8k": CONFIGS["c2_8k"],
        "c2_4k_det": CONFIGS["c2_4k"].with_(name=CONFIGS["c2_4k"].name + "_det", deterministic=True, engine=0),
        "c2_8k_det": CONFIGS["c2_8k"].with_(name=CONFIGS["c2_8k"].name + "_det", deterministic=True, engine=0),
        "c4": CONFIGS["c4"],
        "c4_f16": CONFIGS["c4_f16"],
        "c5": CONFIGS["c5"],
        "nonsquare": CONFIGS["nonsquare"],
    }


def main_kernel_bytes(w) -> int:
    """Algorithmic HBM bytes of one launch of the streaming kernel: Q, dO and
    O read and dQ written once per query-head row, plus the row's LSE (fp32)
    -- it forms delta itself; with a sink it reads delta (fp32) instead of O;
    K, V read and dK, dV written once per kv-head row."""
    rows_q = sum(w.valid_len_q()) * w.heads_q
    rows_kv = sum(w.valid_len_kv()) * w.heads_kv
    per_q = 3 * w.head_dim * 2 + 8 if w.sink else 4 * w.head_dim * 2 + 4
    return rows_q * per_q + rows_kv * (4 * w.head_dim * 2)


def compulsory_bytes(w) -> int:
    """Compulsory HBM bytes of one backward: Q, O, dO read and dQ written per
    query-head row, K, V read and dK, dV written per kv-head row (16-bit),
    plus the row's LSE (fp32)."""
    rows_q = sum(w.valid_len_q()) * w.heads_q
    rows_kv = sum(w.valid_len_kv()) * w.heads_kv
    return rows_q * (4 * w.head_dim * 2 + 4) + rows_kv * (4 * w.head_dim * 2)


def roofline_fractions(w, ms):
    """(fraction of bf16 MFMA peak, fraction of the attainable roofline,
    bound) of a step of ms milliseconds."""
    from sliding_window_attention_flash_amd.synth import flops
    fl = flops(w)
    tf = fl / (ms * 1e-3) / 1e12
    attainable = min(BF16_MFMA_PEAK_TFLOPS, fl / compulsory_bytes(w) * HBM_PEAK_GBS / 1e3)
    bound = "mfma" if attainable >= BF16_MFMA_PEAK_TFLOPS else "hbm"
    return tf / BF16_MFMA_PEAK_TFLOPS, tf / attainable, bound


def _prepare(w, seed):
    import torch  # noqa: F401
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
                      engine=w.engine, sink=inp["sink"], **mk)
    return inp, fw, o, lse, bw


def _median(xs):
    ys = sorted(xs)
    n = len(ys)
    return ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])


def time_workload(w, steps, warmup, repeats=3, seed=0, forward=True, main_kernel=False, min_warm_s=0.5):
    """Times the backward of workload w by the protocol of the module
    docstring.  Returns a dict: ms (median over repeats of the per-repeat
    median step), per-repeat medians, host_mean_ms, the main kernel's mean
    HIP-event time (main_kernel=True), relay expiries, the forward's time
    per call, and the last repeat's inputs and outputs (for the CPU leg)."""
    import torch

    hip = _hip()

    def events(n):
        ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert hip.hipEventCreate(ctypes.byref(e)) == 0
            ev.append(e)
        return ev

    def elapsed(a, b):
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    res = {"repeat_ms": [], "host_mean_ms": [], "expiries": 0}
    ev = events(steps + 1)
    last = None
    for r in range(repeats):
        inp, fw, o, lse, bw = _prepare(w, seed + r)
        for _ in range(warmup):
            bw.run()
        if r == 0:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < min_warm_s:
                for _ in range(8):
                    bw.run()
                torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        torch.cuda.synchronize()
        hip.hipEventRecord(ev[0], ctypes.c_void_p(stream.cuda_stream))
        for k in range(steps):
            bw.run()
            hip.hipEventRecord(ev[k + 1], ctypes.c_void_p(stream.cuda_stream))
        torch.cuda.synchronize()
        res["repeat_ms"].append(_median([elapsed(ev[k], ev[k + 1]) for k in range(steps)]))
        # the same number of steps timed as a whole, without events
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            bw.run()
        torch.cuda.synchronize()
        res["host_mean_ms"].append((time.perf_counter() - t0) / steps * 1e3)
        if w.deterministic:
            res["expiries"] += bw.relay_expiries()
        last = (inp, o, lse, bw)
    for e in ev:
        hip.hipEventDestroy(e)
    res["ms"] = _median(res["repeat_ms"])
    inp, o, lse, bw = last
    # the last repeat's backward outputs on its inputs, for the CPU leg
    dq, dk, dv, dsink = bw.run()
    torch.cuda.synchronize()
    res["last"] = dict(inp=inp, o=o, lse=lse, dq=dq, dk=dk, dv=dv, dsink=dsink)
    if main_kernel:
        # events right around the main kernel of each step (extra stream
        # packets, so these steps are not the timed ones); they are the
        # main kernel's last dispatches of the run (profile summaries rely
        # on that)
        mev = events(2 * steps)
        for k in range(steps):
            bw.run_events(mev[2 * k].value, mev[2 * k + 1].value)
        torch.cuda.synchronize()
        res["main_ms"] = sum(elapsed(mev[2 * k], mev[2 * k + 1]) for k in range(steps)) / steps
        for e in mev:
            hip.hipEventDestroy(e)
    if forward:
        fwd = _forward_of(w, inp)
        for _ in range(max(3, warmup)):
            fwd.run()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fwd.run()
        torch.cuda.synchronize()
        res["forward_ms"] = (time.perf_counter() - t0) / steps * 1e3
    return res


def _forward_of(w, inp):
    from sliding_window_attention_flash_amd import api
    mk = dict(causal=w.causal, bottom_right=w.bottom_right, window_left=w.window_left,
              window_right=w.window_right, scale=w.softmax_scale, cu_seqlens_q=inp["cu_seqlens_q"],
              cu_seqlens_kv=inp["cu_seqlens_kv"], seq_lens_q=inp["seq_lens_q"], seq_lens_kv=inp["seq_lens_kv"])
    if w.layout == "thd":
        mk.update(max_seqlen_q=w.seq_q, max_seqlen_kv=w.seq_kv)
    return api.Forward(inp["q"], inp["k"], inp["v"], sink=inp["sink"], **mk)


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
    """HBM bytes per dispatch of every backward kernel in two rocprofv3
    --pmc runs (FETCH_SIZE, then WRITE_SIZE), each counter divided by what it
    reads per byte moved by the calibration copy.  The TRAFFIC record (what
    the JSON line's roofline.traffic reads) is written for the dominant
    kernel of the default workload when it ran."""
    w = workloads()[workload]
    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")
    _, cf = _pick(fetch, COPY_KERNEL)
    _, cw = _pick(write, COPY_KERNEL)
    copy_kib = COPY_BYTES / 1024
    ff, fw = cf / copy_kib, cw / copy_kib  # counter KiB per byte-KiB moved
    lines = [f"# HBM traffic per kernel, workload {w.name}", "",
             "commands (FETCH_SIZE pass, then WRITE_SIZE pass):", *[f"    {c}" for c in command], "",
             f"calibration copy of {COPY_BYTES} bytes ({COPY_KERNEL}): FETCH_SIZE {cf:.1f} KiB, "
             f"WRITE_SIZE {cw:.1f} KiB",
             f"factors (counter bytes per byte moved): fetch {ff:.4f}, write {fw:.4f}", "",
             f"{'kernel':20s} {'launches':>8s} {'fetch MB':>10s} {'write MB':>10s} {'total MB':>10s}"]
    rec = None
    total = 0.0
    for k in SQ_KERNELS:
        try:
            nf, kf = _pick(fetch, k)
            nw, kw = _pick(write, k)
        except RuntimeError:
            continue
        fb, wb = kf * 1024 / ff, kw * 1024 / fw
        total += fb + wb if not k.startswith("fwd") else 0.0  # (the forward is not part of the step)
        lines.append(f"{k:20s} {nf:8d} {fb / 1e6:10.2f} {wb / 1e6:10.2f} {(fb + wb) / 1e6:10.2f}")
        if k == MAIN_KERNEL:
            algo = main_kernel_bytes(w)
            rec = {"kernel": MAIN_KERNEL, "workload": w.name, "launches_fetch": nf, "launches_write": nw,
                   "fetch_kib_per_launch": kf, "write_kib_per_launch": kw, "copy_bytes": COPY_BYTES,
                   "copy_fetch_kib": cf, "copy_write_kib": cw, "fetch_factor": ff, "write_factor": fw,
                   "traffic_bytes_per_launch": fb + wb, "algorithmic_bytes_per_launch": algo,
                   "source_sha256": kernel_source_hash()}
    comp = compulsory_bytes(w)
    lines += ["", f"backward kernels together   {total / 1e6:10.2f} MB per step; compulsory bytes "
                  f"{comp / 1e6:.2f} MB (traffic / compulsory = {total / comp:.3f})"]
    if rec:
        lines += [f"{MAIN_KERNEL}: algorithmic bytes {rec['algorithmic_bytes_per_launch'] / 1e6:.2f} MB "
                  f"(traffic / algorithmic = {rec['traffic_bytes_per_launch'] / rec['algorithmic_bytes_per_launch']:.3f})",
                  "", "TRAFFIC " + json.dumps(rec)]
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


SQ_KERNELS = ("bwd_stream_kernel", "bwd_qstream_kernel", "bwd_qstream_fix_kernel", "bwd_main_kernel", "bwd_dq_kernel",
              "bwd_dot_kernel", "bwd_clear_kernel", "bwd_dsink_kernel", "fwd_qstream_kernel", "fwd_kernel")
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


# oracle work (attended pairs x head_dim x query heads) above which the CPU
# leg checks whole batch entries instead of the whole dense workload: about
# 8 s of oracle time on 16 host threads
ORACLE_FULL_WORK = 1.2e10


def _leading(w, n):
    """Workload w cut to its first n batch entries or packed sequences."""
    if w.layout == "thd":
        return w.with_(name=f"{w.name}_s0-{n - 1}", batch=n, len_q=w.len_q[:n], len_kv=w.len_kv[:n],
                       cap_q=w.cap_q[:n], cap_kv=w.cap_kv[:n], seq_q=max(w.cap_q[:n]),
                       seq_kv=max(w.cap_kv[:n]))
    return w.with_(name=f"{w.name}_b0-{n - 1}", batch=n,
                   pad_len_q=w.pad_len_q[:n] if w.pad_len_q else None,
                   pad_len_kv=w.pad_len_kv[:n] if w.pad_len_kv else None)


def cpu_leg(w, last):
    """The fp64 oracle on the inputs of the workload's last timed repeat:
    its wall time and the per-gradient parity errors of the GPU outputs.
    Workloads too large for one oracle run are checked on their leading
    batch entries or packed sequences (as many as fit ORACLE_FULL_WORK, at
    least one)."""
    import oracle
    import torch
    from sliding_window_attention_flash_amd.synth import attended_pairs_per_head

    def work(wx):
        return attended_pairs_per_head(wx) * wx.heads_q * wx.head_dim

    # the leading batch entries (dense) or packed sequences that fit the
    # budget, at least one; rows [0, nq) / [0, nk) of the packed tensors
    nb = w.batch
    if work(w) > ORACLE_FULL_WORK:
        nb = 1
        while nb < w.batch and work(_leading(w, nb + 1)) <= ORACLE_FULL_WORK:
            nb += 1
    ws = w if nb == w.batch else _leading(w, nb)
    nq = sum(ws.cap_q) if w.layout == "thd" else nb
    nk = sum(ws.cap_kv) if w.layout == "thd" else nb
    inp = last["inp"]
    cpu = {k: inp[k][:(nk if k in ("k", "v") else nq)].cpu() for k in ("q", "k", "v", "dO")}
    sink = inp["sink"].cpu() if inp["sink"] is not None else None
    p = oracle.Problem.for_workload(ws)
    t0 = time.perf_counter()
    ref = oracle.backward(p, cpu["q"], cpu["k"], cpu["v"], cpu["dO"], sink)
    dt = time.perf_counter() - t0
    errs = {}
    pairs = [("dQ", "dq", "dq"), ("dK", "dk", "dk"), ("dV", "dv", "dv")]
    if w.sink and ws is w:  # dSink sums over every sequence
        pairs.append(("dSink", "dsink", "dsink"))
    for name, gk, rk in pairs:
        g = last[gk]
        if name != "dSink":
            g = g[:(nk if name in ("dK", "dV") else nq)]
        g = g.double().cpu().reshape(-1)
        r = ref[rk].reshape(-1)
        rn, rmax = float(r.norm()), float(r.abs().max())
        d = g - r
        errs[name] = {"rel_fro": float(d.norm()) / rn if rn else float(g.abs().max()),
                      "max_abs_over_max_ref": float(d.abs().max()) / rmax if rmax else float(g.abs().max()),
                      "nan": bool(torch.isnan(g).any())}
    units = ws.batch * ws.heads_kv
    sample_pairs = attended_pairs_per_head(ws) * ws.heads_q
    what = "packed sequences" if w.layout == "thd" else "batch entries"
    return {"oracle_ms": dt * 1e3, "cores": min(oracle.num_threads(), units),
            "sample": ("whole workload" if ws is w else f"{what} 0..{nb - 1} of {w.batch}")
                      + f": {sample_pairs} attended pairs, fp64 forward + backward",
            "oracle_tflops": 10.0 * ws.head_dim * sample_pairs / dt / 1e12,
            "parity": errs}


def workload_entry(w, t):
    from sliding_window_attention_flash_amd.synth import flops
    fl = flops(w)
    f_peak, f_roof, bound = roofline_fractions(w, t["ms"])
    e = {"workload": w.name, "ms": t["ms"], "tflops": fl / (t["ms"] * 1e-3) / 1e12,
         "repeat_ms": t["repeat_ms"], "host_mean_ms": _median(t["host_mean_ms"]),
         "frac_bf16_mfma_peak": f_peak, "frac_attainable_roofline": f_roof, "roofline_bound": bound,
         "compulsory_bytes": compulsory_bytes(w), "attended_flops": fl, "relay_expiries": t["expiries"]}
    if "forward_ms" in t:
        e["forward_ms"] = t["forward_ms"]
        e["forward_tflops"] = 0.4 * fl / (t["forward_ms"] * 1e-3) / 1e12
    if "main_ms" in t:
        e["main_ms"] = t["main_ms"]
    return e


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--repeats", type=int, default=3)
    ap.add_argument("--warm-seconds", type=float, default=0.5,
                    help="backward steps run before each workload's first repeat, in seconds of wall time")
    ap.add_argument("--workload", default="c3", choices=sorted(workloads()))
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU leg (oracle time and parity errors)")
    ap.add_argument("--no-extra", action="store_true", help="time the headline workload only")
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

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    wl = workloads()
    w = wl[args.workload]
    t = time_workload(w, args.steps, args.warmup, args.repeats, main_kernel=True, min_warm_s=args.warm_seconds)
    head = workload_entry(w, t)
    nbytes = main_kernel_bytes(w)
    achieved = nbytes / (t["main_ms"] * 1e-3) / 1e9
    extra = {"timing": f"median over {args.repeats} repeats (fresh tensors each) of the median of "
                       f"{args.steps} per-step HIP-event times, after {args.warmup} warm-up steps and "
                       f"at least {args.warm_seconds} s of backward steps",
             "main_kernel": MAIN_KERNEL, "main_kernel_ms": t["main_ms"],
             "main_kernel_algorithmic_bytes": nbytes,
             "main_kernel_attended_tflops": head["attended_flops"] / (t["main_ms"] * 1e-3) / 1e12,
             "headline": head}
    line = {
        "metric": METRIC, "value": head["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "repeats": args.repeats, "ms_per_step": t["ms"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads_q": w.heads_q, "heads_kv": w.heads_kv,
                   "head_dim": w.head_dim, "seq_len": w.seq_q, "window_left": w.window_left,
                   "mask": "causal_bottom_right" if w.bottom_right else "causal_top_left",
                   "dq_mode": {1: "fp32 atomics"}.get(w.engine, "ordered relay" if w.deterministic else "plan's choice")},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": stored_traffic(w)},
        "extra": extra,
    }
    if not args.no_cpu_baseline:
        c = cpu_leg(w, t["last"])
        head["oracle"] = {k: c[k] for k in ("oracle_ms", "cores", "sample")}
        head["parity"] = c["parity"]
        line["cpu_baseline"] = {"value": c["oracle_tflops"], "unit": "TFLOP/s", "cores": c["cores"],
                                "kind": "oracle", "sample": c["sample"] + f" of {w.name}, "
                                f"{c['oracle_ms'] / 1e3:.2f} s"}
    del t
    if not args.no_extra:
        for name in ("c3_atomic", "c1", "c2_4k", "c2_8k", "c2_4k_det", "c2_8k_det", "c4", "c4_f16", "c5",
                     "nonsquare"):
            if name == args.workload:
                continue
            wx = wl[name]
            tx = time_workload(wx, args.steps, args.warmup, args.repeats, min_warm_s=args.warm_seconds)
            e = workload_entry(wx, tx)
            if not args.no_cpu_baseline:
                c = cpu_leg(wx, tx["last"])
                e["oracle"] = {k: c[k] for k in ("oracle_ms", "cores", "sample")}
                e["parity"] = c["parity"]
            extra[name] = e
            del tx
            torch.cuda.empty_cache()
    print(json.dumps(line), flush=True)
    if args.copy_calibration:
        copy_calibration()


if __name__ == "__main__":
    main()
