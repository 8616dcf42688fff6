"""Measured study behind the plan's engine table: which backward kernels and
dQ mechanism to run for a shape the streaming kernel applies to
(multi-head, causal, left window up to 128 keys, head_dim 64).

    python -m sliding_window_attention_flash_amd.engine_study [--out FILE]

For a grid of batch x heads, sequence lengths, windows and both anchors it
times the backward step with each engine forced through the descriptor's
``engine`` field -- 1 streaming kernel with fp32 atomics at chunk
boundaries, 2 streaming kernel with the chunk relay, 3 per-tile kernels with
the q-major dQ pass -- in interleaved rounds, and prints the medians, the
fastest engine for deterministic = 0 (any) and for deterministic = 1
(engines 2 and 3), and what the plan's default (engine 0) picked.  Inputs
are the seeded synthetic ones of ``synth``.
"""
from __future__ import annotations

import argparse
import statistics
import sys
import time

import torch

from . import api
from .synth import Workload, make_inputs

ENGINES = (1, 2, 3)


def _mask_kw(w: Workload) -> dict:
    return dict(causal=w.causal, bottom_right=w.bottom_right, window_left=w.window_left,
                window_right=w.window_right, scale=w.softmax_scale)


def _time(fn, iters: int, warmup: int) -> float:
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(iters):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / iters * 1e3


def grid():
    out = []
    for (b, h) in ((1, 2), (2, 16), (8, 16)):
        for s in (1024, 4096, 16384):
            for win in (64, 128):
                out.append(Workload(f"b{b}_h{h}_s{s}_w{win}_tl", torch.bfloat16, b, h, h, 64, s, s,
                                    window_left=win, scale=0.125))
    for (sq, skv) in ((4096, 4096), (1024, 8192)):
        out.append(Workload(f"b2_h16_q{sq}_kv{skv}_w128_br", torch.bfloat16, 2, 16, 16, 64, sq, skv,
                            bottom_right=True, window_left=128, scale=0.125))
    return out


def study(workloads, rounds: int = 3, iters: int = 10, warmup: int = 5):
    rows = []
    for w in workloads:
        inp = make_inputs(w, device="cuda", seed=0)
        o, lse = api.Forward(inp["q"], inp["k"], inp["v"], **_mask_kw(w)).run()
        times = {(e, d): [] for e in (0,) + ENGINES for d in (0, 1)}
        for _ in range(rounds):
            for (e, d) in times:
                if (e, d) == (1, 1):  # atomics are not repeatable
                    continue
                bw = api.Backward(inp["q"], inp["k"], inp["v"], o, inp["dO"], lse, engine=e, deterministic=d,
                                  **_mask_kw(w))
                times[(e, d)].append(_time(bw.run, iters, warmup))
        med = {k: statistics.median(v) for k, v in times.items() if v}
        rows.append((w, med))
        print(f"  {w.name}: " + ", ".join(f"engine {e} det {d}: {t:.4f}" for (e, d), t in sorted(med.items())),
              flush=True)
        del inp, o, lse
        torch.cuda.empty_cache()
    return rows


def report(rows) -> list:
    lines = ["workload                   engine 1   engine 2   engine 3 | det 0: best  default  default/best"
             " | det 1: best  default  default/best"]
    for w, m in rows:
        b0 = min(ENGINES, key=lambda e: m[(e, 0)])
        b1 = min((2, 3), key=lambda e: m[(e, 1)])
        lines.append(f"{w.name:26s} " + " ".join(f"{m[(e, 0)]:9.4f}" for e in ENGINES)
                     + f"  |        {b0}  {m[(0, 0)]:8.4f}  {m[(0, 0)] / m[(b0, 0)]:6.3f}"
                     + f"        |        {b1}  {m[(0, 1)]:8.4f}  {m[(0, 1)] / m[(b1, 1)]:6.3f}")
    return lines


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out")
    args = ap.parse_args()
    if not torch.cuda.is_available():
        print("engine_study needs a GPU", file=sys.stderr)
        sys.exit(1)
    lines = ["# engine study: median ms per backward step, engines forced through the descriptor",
             "# (1 streaming + fp32 atomics, 2 streaming + chunk relay, 3 per-tile + q-major dQ pass);",
             "# engine columns at deterministic 0; 'default' is the plan's own choice (engine 0)",
             "", "command: python -m sliding_window_attention_flash_amd.engine_study"
             + (f" --out {args.out}" if args.out else ""), ""]
    lines += report(study(grid()))
    text = "\n".join(lines) + "\n"
    print(text, flush=True)
    if args.out:
        with open(args.out, "w") as fh:
            fh.write(text)


if __name__ == "__main__":
    main()
