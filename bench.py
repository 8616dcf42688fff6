"""Benchmark of the sliding-window attention backward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload c3|c3_atomic|c2_4k|c2_8k]

A step is one full backward, sdpa_bwd_run: the dot preprocess, the main
window-bounded kernel with its dQ accumulation (ordered relay or fp32
atomics), the dQ conversion (atomic mode) and dSink (with sinks), on inputs
already resident in HBM.  The default workload is the long-sequence one the
target names: batch 2, 16 heads, head_dim 64, S = 32768, causal top-left with
a left window of 128, bf16, deterministic relay.  Prints one JSON line.

FLOPs count attended (query, key) pairs only: 10 * head_dim per pair per
query head.  The roofline entry is for the dominant kernel (bwd_main), timed
with HIP events recorded on its launch stream around every launch.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
METRIC = "SWA backward ms & TFLOP/s (attended pairs), b2 h16 d64 W128 S=4k/8k/32k"


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
        "c2_4k": CONFIGS["c2_4k"],
        "c2_8k": CONFIGS["c2_8k"],
    }


def main_kernel_bytes(w) -> int:
    """Algorithmic HBM bytes of one bwd_main launch: Q, dO read and dQ
    written once per query-head row, plus the row's LSE and delta (fp32);
    K, V read and dK, dV written once per kv-head row."""
    from sliding_window_attention_flash_amd.synth import Workload  # noqa: F401
    rows_q = sum(w.valid_len_q()) * w.heads_q
    rows_kv = sum(w.valid_len_kv()) * w.heads_kv
    return rows_q * (3 * w.head_dim * 2 + 8) + rows_kv * (4 * w.head_dim * 2)


def time_backward(w, steps, warmup, seed=0):
    import torch
    from sliding_window_attention_flash_amd import api
    from sliding_window_attention_flash_amd.synth import make_inputs

    inp = make_inputs(w, device="cuda", seed=seed)
    mk = dict(causal=w.causal, bottom_right=w.bottom_right, window_left=w.window_left,
              scale=w.softmax_scale)
    o, lse = api.forward(inp["q"], inp["k"], inp["v"], sink=inp["sink"], **mk)
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
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        bw.run_events(ev[2 * s].value, ev[2 * s + 1].value)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    main_ms = []
    for s in range(steps):
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), ev[2 * s], ev[2 * s + 1]) == 0
        main_ms.append(ms.value)
    for e in ev:
        hip.hipEventDestroy(e)
    expiries = bw.relay_expiries() if w.deterministic else 0
    return wall * 1e3, sum(main_ms) / len(main_ms), expiries


def cpu_baseline(w):
    """The fp64 oracle's backward timed on a bounded slice of the workload
    (batch 0, one query head per host thread, each with its own kv head so
    the oracle's (sequence, kv head) units spread over every thread), scaled
    to attended TFLOP/s."""
    import oracle
    from sliding_window_attention_flash_amd.synth import make_inputs

    budget_heads = max(1, min(oracle.num_threads(), w.heads_q))
    ws = w.with_(batch=1, heads_q=budget_heads, heads_kv=budget_heads, name=w.name + "_slice")
    inp = make_inputs(ws, device="cpu", seed=0)
    p = oracle.Problem.dense(1, budget_heads, budget_heads, w.seq_q, w.seq_kv, w.head_dim,
                             causal=w.causal, bottom_right=w.bottom_right,
                             window_left=w.window_left, scale=w.softmax_scale)
    t0 = time.perf_counter()
    oracle.backward(p, inp["q"], inp["k"], inp["v"], inp["dO"], None)
    dt = time.perf_counter() - t0
    pairs = oracle.attended_pairs(p) * budget_heads
    flops = 10.0 * w.head_dim * pairs
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": min(oracle.num_threads(), budget_heads),
            "kind": "oracle",
            "sample": f"fp64 oracle backward (forward recompute included) on batch 0, "
                      f"{budget_heads} head(s) of {w.name}: {pairs} attended pairs in {dt:.2f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c3", choices=sorted(workloads()))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the 4k / 8k / atomic side timings")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              "(the per-GPU kernel is the one-GPU workload; see DESIGN.md for how it would shard)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from sliding_window_attention_flash_amd.synth import flops

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    wl = workloads()
    w = wl[args.workload]
    ms, main_ms, exp = time_backward(w, args.steps, args.warmup)
    fl = flops(w)
    tflops = fl / (ms * 1e-3) / 1e12
    nbytes = main_kernel_bytes(w)
    achieved = nbytes / (main_ms * 1e-3) / 1e9
    extra = {"main_kernel_ms": main_ms, "main_kernel_attended_tflops": fl / (main_ms * 1e-3) / 1e12,
             "frac_bf16_mfma_peak": tflops / BF16_MFMA_PEAK_TFLOPS, "relay_expiries": exp,
             "attended_flops": fl}
    if not args.no_extra:
        for name in ("c3_atomic", "c2_4k", "c2_8k"):
            if name == args.workload:
                continue
            m2, mm2, _ = time_backward(wl[name], max(5, args.steps // 2), 3)
            extra[name] = {"ms": m2, "tflops": flops(wl[name]) / (m2 * 1e-3) / 1e12, "main_ms": mm2}
    line = {
        "metric": METRIC, "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads_q": w.heads_q, "heads_kv": w.heads_kv,
                   "head_dim": w.head_dim, "seq_len": w.seq_q, "window_left": w.window_left,
                   "mask": "causal_bottom_right" if w.bottom_right else "causal_top_left",
                   "dq_mode": "relay" if w.deterministic else "atomic"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None},
        "extra": extra,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
