"""Measured study behind the plan's q-run table: how many consecutive 64-row
q-tiles one block of the q-major passes (the forward, and the unordered dQ
pass of the per-tile backward) should walk.

    python -m sliding_window_attention_flash_amd.tile_study [--out FILE]

For GQA problems (32 query / 4 kv heads, batch 2, S = 8192, bottom-right)
over head_dim {64, 128} and left windows from 32 to 2048 keys, it times the
backward step and the forward with runs of 1, 2, 4 and 8 q-tiles
(``q_run_tiles``) and with the plan's default (0), in interleaved rounds,
and prints the medians with the best run marked.  Inputs are the seeded
synthetic ones of ``synth``.
"""
from __future__ import annotations

import argparse
import statistics
import sys
import time

import torch

from . import api
from .synth import Workload, make_inputs

RUNS = (0, 1, 2, 4, 8)  # 0: the plan's default


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


def study(workloads, rounds: int = 3, iters: int = 5, warmup: int = 3):
    rows = []
    for w in workloads:
        inp = make_inputs(w, device="cuda", seed=0)
        o, lse = api.Forward(inp["q"], inp["k"], inp["v"], **_mask_kw(w)).run()
        bwd = {r: [] for r in RUNS}
        fwd = {r: [] for r in RUNS}
        for _ in range(rounds):
            for r in RUNS:
                fw = api.Forward(inp["q"], inp["k"], inp["v"], q_run_tiles=r, **_mask_kw(w))
                bw = api.Backward(inp["q"], inp["k"], inp["v"], o, inp["dO"], lse, q_run_tiles=r, **_mask_kw(w))
                fwd[r].append(_time(fw.run, iters, warmup))
                bwd[r].append(_time(bw.run, iters, warmup))
        med_b = {r: statistics.median(v) for r, v in bwd.items()}
        med_f = {r: statistics.median(v) for r, v in fwd.items()}
        rows.append((w, med_b, med_f))
        print(f"  {w.name}: backward {med_b[0]:.4f} ms, forward {med_f[0]:.4f} ms (default run)", flush=True)
        del inp, o, lse
        torch.cuda.empty_cache()
    return rows


def report(rows) -> list:
    lines = ["workload                 pass      default   " + "  ".join(f"run {r:<5d}" for r in RUNS[1:])
             + "  best  default/best"]
    for w, mb, mf in rows:
        for name, m in (("backward", mb), ("forward", mf)):
            best = min(RUNS[1:], key=lambda r: m[r])
            lines.append(f"{w.name:24s} {name:8s}  {m[0]:8.4f}  " + "  ".join(f"{m[r]:9.4f}" for r in RUNS[1:])
                         + f"  {best:4d}  {m[0] / m[best]:.3f}")
    return lines


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out")
    args = ap.parse_args()
    if not torch.cuda.is_available():
        print("tile_study needs a GPU", file=sys.stderr)
        sys.exit(1)
    wls = [Workload(f"gqa32x4_d{d}_w{win}_s8192", torch.bfloat16, 2, 32, 4, d, 8192, 8192, bottom_right=True,
                    window_left=win)
           for d in (64, 128) for win in (32, 64, 128, 256, 512, 1024, 2048)]
    lines = ["# q-run study: median ms per call (backward step, forward) for runs of q-tiles per block",
             "", "command: python -m sliding_window_attention_flash_amd.tile_study"
             + (f" --out {args.out}" if args.out else ""), ""]
    lines += report(study(wls))
    text = "\n".join(lines) + "\n"
    print(text, flush=True)
    if args.out:
        with open(args.out, "w") as fh:
            fh.write(text)


if __name__ == "__main__":
    main()
