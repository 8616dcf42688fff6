"""Measured studies behind the plan's engine table: which backward kernels
and dQ mechanism to run for a shape more than one engine applies to.

    python -m sliding_window_attention_flash_amd.engine_study [--family F] [--out FILE]

Family ``mha_d64`` (the default): multi-head, causal, left window up to 128
keys, head_dim 64, where the streaming kernel applies -- engines 1
(streaming kernel, fp32 atomics at chunk boundaries), 2 (streaming kernel,
chunk relay) and 3 (per-tile kernels, q-major dQ pass).  Family ``d128``:
head_dim 128, causal, left window up to 96 keys, GQA and multi-head, where
the q-major streaming kernel applies -- engines 3 and 5.  Family
``fwd_d128``: the forward on head_dim 128, causal, left window up to 96
keys, query-head groups of a multiple of 8 -- the per-tile forward (engine 3
on the forward plan) and the q-major forward (engine 5).

For each shape of the family's grid it times the backward step (or the
forward) with each engine forced through the descriptor's ``engine`` field,
in interleaved rounds, and prints the medians, the fastest engine for
deterministic = 0 (any) and for deterministic = 1 (the repeatable engines),
and what the plan's default (engine 0) picked.  Inputs are the seeded
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

# per family: the engines timed, the repeatable ones among them
FAMILIES = {"mha_d64": ((1, 2, 3), (2, 3)), "d128": ((3, 5), (3, 5)), "fwd_d128": ((3, 5), (3, 5))}


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


def grid(family: str):
    out = []
    if family == "mha_d64":
        for (b, h) in ((1, 2), (2, 16), (8, 16)):
            for s in (1024, 4096, 16384):
                for win in (64, 128):
                    out.append(Workload(f"b{b}_h{h}_s{s}_w{win}_tl", torch.bfloat16, b, h, h, 64, s, s,
                                        window_left=win, scale=0.125))
        for (sq, skv) in ((4096, 4096), (1024, 8192)):
            out.append(Workload(f"b2_h16_q{sq}_kv{skv}_w128_br", torch.bfloat16, 2, 16, 16, 64, sq, skv,
                                bottom_right=True, window_left=128, scale=0.125))
        return out
    if family == "fwd_d128":
        # groups of 8 and 16, both anchors, windows 0 to 96, 1 to 72
        # (sequence, kv head) pairs, 1K to 16K rows, with and without a sink
        for (b, hq, hkv) in ((1, 8, 1), (2, 16, 2), (2, 32, 2), (12, 48, 6)):
            for s in (1024, 4096, 16384):
                for win in (0, 32, 96):
                    if b * hq * s > 12 * 48 * 16384 // 2 and win != 96:
                        continue
                    out.append(Workload(f"b{b}_h{hq}x{hkv}_s{s}_w{win}_tl", torch.bfloat16, b, hq, hkv, 128, s, s,
                                        window_left=win))
        out.append(Workload("b12_h48x6_s16484_w96_br", torch.bfloat16, 12, 48, 6, 128, 16484, 16484,
                            bottom_right=True, window_left=96))
        out.append(Workload("b4_h32x4_q2048_kv4096_w64_br_f16", torch.float16, 4, 32, 4, 128, 2048, 4096,
                            bottom_right=True, window_left=64))
        for (b, hq, hkv, s) in ((1, 8, 1, 4096), (12, 48, 6, 4096)):
            out.append(Workload(f"b{b}_h{hq}x{hkv}_s{s}_w96_br_sink", torch.bfloat16, b, hq, hkv, 128, s, s,
                                bottom_right=True, window_left=96, sink=True))
        return out
    # head_dim 128: GQA groups of 8 and multi-head, small to full-chip grids
    for (b, hq, hkv) in ((1, 2, 2), (1, 8, 1), (2, 16, 2), (2, 16, 16), (12, 48, 6)):
        for s in (1024, 4096, 8192, 16384):
            for win in (32, 96):
                if b * hq * s > 12 * 48 * 16384 // 2 and win != 96:
                    continue
                if s == 8192 and (b, hq, hkv) != (2, 16, 2):
                    continue
                out.append(Workload(f"b{b}_h{hq}x{hkv}_s{s}_w{win}_tl", torch.bfloat16, b, hq, hkv, 128, s, s,
                                    window_left=win))
    out.append(Workload("b12_h48x6_s16484_w96_br", torch.bfloat16, 12, 48, 6, 128, 16484, 16484,
                        bottom_right=True, window_left=96))
    out.append(Workload("b4_h32x4_q2048_kv4096_w96_br_f16", torch.float16, 4, 32, 4, 128, 2048, 4096,
                        bottom_right=True, window_left=96))
    # with sink logits
    for (b, hq, hkv, s) in ((1, 8, 1, 4096), (2, 16, 2, 1024), (2, 16, 2, 4096)):
        out.append(Workload(f"b{b}_h{hq}x{hkv}_s{s}_w32_tl_sink", torch.bfloat16, b, hq, hkv, 128, s, s,
                            window_left=32, sink=True))
    out.append(Workload("b12_h48x6_s4096_w96_br_sink", torch.bfloat16, 12, 48, 6, 128, 4096, 4096,
                        bottom_right=True, window_left=96, sink=True))
    return out


def study(workloads, engines, rounds: int = 3, iters: int = 10, warmup: int = 5):
    rows = []
    for w in workloads:
        inp = make_inputs(w, device="cuda", seed=0)
        o, lse = api.Forward(inp["q"], inp["k"], inp["v"], sink=inp["sink"], **_mask_kw(w)).run()
        times = {(e, d): [] for e in (0,) + engines for d in (0, 1)}
        for _ in range(rounds):
            for (e, d) in times:
                if (e, d) == (1, 1):  # atomics are not repeatable
                    continue
                bw = api.Backward(inp["q"], inp["k"], inp["v"], o, inp["dO"], lse, engine=e, deterministic=d,
                                  sink=inp["sink"], **_mask_kw(w))
                times[(e, d)].append(_time(bw.run, iters, warmup))
        med = {k: statistics.median(v) for k, v in times.items() if v}
        rows.append((w, med))
        print(f"  {w.name}: " + ", ".join(f"engine {e} det {d}: {t:.4f}" for (e, d), t in sorted(med.items())),
              flush=True)
        del inp, o, lse
        torch.cuda.empty_cache()
    return rows


def study_forward(workloads, engines, rounds: int = 3, iters: int = 10, warmup: int = 5):
    rows = []
    for w in workloads:
        inp = make_inputs(w, device="cuda", seed=0)
        fws = {e: api.Forward(inp["q"], inp["k"], inp["v"], sink=inp["sink"], engine=e, **_mask_kw(w))
               for e in (0,) + engines}
        times = {e: [] for e in fws}
        for _ in range(rounds):
            for e, fw in fws.items():
                times[e].append(_time(fw.run, iters, warmup))
        med = {e: statistics.median(v) for e, v in times.items()}
        rows.append((w, med))
        print(f"  {w.name}: " + ", ".join(f"engine {e}: {t:.4f}" for e, t in sorted(med.items())), flush=True)
        del inp, fws
        torch.cuda.empty_cache()
    return rows


def report_forward(rows, engines) -> list:
    lines = [f"{'workload':34s}" + "".join(f"  engine {e}" for e in engines) + " | best  default  default/best"]
    for w, m in rows:
        b = min(engines, key=lambda e: m[e])
        lines.append(f"{w.name:34s} " + " ".join(f"{m[e]:9.4f}" for e in engines)
                     + f"  |    {b}  {m[0]:8.4f}  {m[0] / m[b]:6.3f}")
    return lines


def report(rows, engines, repeatable) -> list:
    lines = [f"{'workload':34s}" + "".join(f"  engine {e}" for e in engines)
             + " | det 0: best  default  default/best | det 1: best  default  default/best"]
    for w, m in rows:
        b0 = min(engines, key=lambda e: m[(e, 0)])
        b1 = min(repeatable, key=lambda e: m[(e, 1)])
        lines.append(f"{w.name:34s} " + " ".join(f"{m[(e, 0)]:9.4f}" for e in engines)
                     + f"  |        {b0}  {m[(0, 0)]:8.4f}  {m[(0, 0)] / m[(b0, 0)]:6.3f}"
                     + f"        |        {b1}  {m[(0, 1)]:8.4f}  {m[(0, 1)] / m[(b1, 1)]:6.3f}")
    return lines


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--family", choices=sorted(FAMILIES), default="mha_d64")
    ap.add_argument("--out")
    args = ap.parse_args()
    if not torch.cuda.is_available():
        print("engine_study needs a GPU", file=sys.stderr)
        sys.exit(1)
    engines, repeatable = FAMILIES[args.family]
    command = ("command: python -m sliding_window_attention_flash_amd.engine_study"
               + f" --family {args.family}" + (f" --out {args.out}" if args.out else ""))
    if args.family == "fwd_d128":
        lines = ["# forward engine study: median ms per forward, engines forced through the descriptor",
                 "# (3 per-tile forward, 5 q-major forward); 'default' is the plan's own choice (engine 0)",
                 "", command, ""]
        lines += report_forward(study_forward(grid(args.family), engines), engines)
    else:
        names = {1: "streaming + fp32 atomics", 2: "streaming + chunk relay", 3: "per-tile + q-major dQ pass",
                 5: "q-major streaming kernel"}
        lines = ["# engine study: median ms per backward step, engines forced through the descriptor",
                 "# (" + ", ".join(f"{e} {names[e]}" for e in engines) + ");",
                 "# engine columns at deterministic 0; 'default' is the plan's own choice (engine 0)",
                 "", command, ""]
        lines += report(study(grid(args.family), engines), engines, repeatable)
    text = "\n".join(lines) + "\n"
    print(text, flush=True)
    if args.out:
        with open(args.out, "w") as fh:
            fh.write(text)


if __name__ == "__main__":
    main()
