"""Seeded synthetic workloads for the sliding-window attention backward.

This module only describes workloads (shapes, masks, sequence-length mixes)
and draws their random inputs.  It holds none of the attention arithmetic,
so both the GPU path and the fp64 oracle can be fed from it.

Inputs are N(0, 1) draws from torch's seeded generator on the requested
device, rounded to the workload's 16-bit type.  Each tensor gets its own
seed, derived from the workload name, the tensor name and a base seed.

The workloads follow the shapes the source pages measure:
  * cudnn-frontend PR #866 ("bound the SM80 backward q-loop by the sliding
    window ..."), commit message: batch 2, 16 heads, head_dim 64, window 128,
    bf16, causal, S = 4k / 8k (and the 2k..32k dashboard range in "Problem");
  * cudnn-frontend PR #2352 ("lead square A100 backward window graphs from a
    measured study"), Measurement section: bf16 b12 48/6 d128 S 16484
    window 96, f16 b24 28/4 d128 S 128 window 8000, and the non-square
    b12 40/8 d64 q128 kv8960 window 8000 class;
  * cudnn-frontend PR #557 ("GQA/MQA, padding mask, right-band widening, and
    sink-token gradients ..."), Summary: per-sequence lengths and sinks.
"""
from __future__ import annotations

import math
import zlib
from dataclasses import dataclass, field, replace
from typing import List, Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: torch.dtype
    batch: int
    heads_q: int
    heads_kv: int
    head_dim: int
    seq_q: int  # dense length, or the largest slot capacity for packed
    seq_kv: int
    causal: bool = True
    bottom_right: bool = False
    window_left: int = -1
    window_right: int = 0  # causal only: inclusive right band (0: plain causal)
    scale: Optional[float] = None
    deterministic: bool = False
    engine: int = 0  # backward kernels / dQ mechanism: 0 the plan's choice, 1..4 forced
    sink: bool = False
    layout: str = "bhsd"  # "bhsd" ([B,H,S,D]) or "thd" ([T,H,D] packed)
    # packed layout: per-sequence valid lengths and slot capacities
    len_q: Optional[tuple] = None
    len_kv: Optional[tuple] = None
    cap_q: Optional[tuple] = None
    cap_kv: Optional[tuple] = None
    # dense layout with a padding mask: per-batch valid lengths
    pad_len_q: Optional[tuple] = None
    pad_len_kv: Optional[tuple] = None

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.head_dim)

    @property
    def total_q(self) -> int:
        return sum(self.cap_q) if self.layout == "thd" else self.batch * self.seq_q

    @property
    def total_kv(self) -> int:
        return sum(self.cap_kv) if self.layout == "thd" else self.batch * self.seq_kv

    def valid_len_q(self) -> List[int]:
        if self.layout == "thd":
            return list(self.len_q)
        return list(self.pad_len_q) if self.pad_len_q else [self.seq_q] * self.batch

    def valid_len_kv(self) -> List[int]:
        if self.layout == "thd":
            return list(self.len_kv)
        return list(self.pad_len_kv) if self.pad_len_kv else [self.seq_kv] * self.batch

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def _roundup(x: int, m: int) -> int:
    return (x + m - 1) // m * m


def packed_lengths(n_seq: int, q_lo: int, q_hi: int, extra_hi: int, seed: int,
                   q_align: int = 64):
    """Per-sequence lengths for a packed varlen batch: s_q ~ U[q_lo, q_hi],
    s_kv = s_q + U[0, extra_hi]; query slots rounded up to ``q_align`` rows
    (the extra rows are padding), key slots packed tight."""
    g = torch.Generator().manual_seed(seed)
    sq = torch.randint(q_lo, q_hi + 1, (n_seq,), generator=g).tolist()
    extra = torch.randint(0, extra_hi + 1, (n_seq,), generator=g).tolist()
    skv = [a + e for a, e in zip(sq, extra)]
    cap_q = [_roundup(a, q_align) for a in sq]
    return tuple(sq), tuple(skv), tuple(cap_q), tuple(skv)


def _c5() -> Workload:
    lq, lk, cq, ck = packed_lengths(8, 64, 512, 8832, seed=5005)
    return Workload("c5_thd_sink_gqa40x8_d64_br_w8000_f16", torch.float16, 8, 40, 8, 64,
                    max(cq), max(ck), causal=True, bottom_right=True, window_left=8000,
                    sink=True, layout="thd", len_q=lq, len_kv=lk, cap_q=cq, cap_kv=ck)


CONFIGS = {
    "c1": Workload("c1_tiny_b1_h2_d64_s256_w64_bf16", torch.bfloat16, 1, 2, 2, 64, 256, 256,
                   window_left=64, scale=0.125),
    # fp32-atomic dQ, as the pages' gpt_oss-style rows are measured
    "c2_4k": Workload("c2_b2_h16_d64_s4096_w128_bf16", torch.bfloat16, 2, 16, 16, 64, 4096, 4096,
                      window_left=128, scale=0.125, engine=1),
    "c2_8k": Workload("c2_b2_h16_d64_s8192_w128_bf16", torch.bfloat16, 2, 16, 16, 64, 8192, 8192,
                      window_left=128, scale=0.125, engine=1),
    "c3": Workload("c3_b2_h16_d64_s32768_w128_bf16_det", torch.bfloat16, 2, 16, 16, 64, 32768,
                   32768, window_left=128, scale=0.125, deterministic=True),
    "c4": Workload("c4_b12_gqa48x6_d128_s16484_br_w96_bf16", torch.bfloat16, 12, 48, 6, 128,
                   16484, 16484, bottom_right=True, window_left=96),
    "c4_f16": Workload("c4_f16_b24_gqa28x4_d128_s128_br_w8000", torch.float16, 24, 28, 4, 128,
                       128, 128, bottom_right=True, window_left=8000),
    "c5": _c5(),
    # the non-square class of the mixed study (PR #2352, opening section):
    # short query, long key sequences under a long window (dtype not stated
    # there; bf16 like the study's first class)
    "nonsquare": Workload("ns_b12_gqa40x8_d64_q128_kv8960_br_w8000_bf16", torch.bfloat16, 12, 40, 8, 64,
                          128, 8960, bottom_right=True, window_left=8000),
}


def _seed(w: Workload, tensor: str, base: int) -> int:
    return (zlib.crc32(f"{w.name}/{tensor}".encode()) ^ (base * 0x9E3779B1)) & 0x7FFFFFFF


def _randn(shape, dtype, device, seed):
    g = torch.Generator(device=device).manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(dtype)


def make_inputs(w: Workload, device="cpu", seed: int = 0) -> dict:
    """Q, K, V, dO (16-bit, N(0,1)), the sink logits (fp32, N(0,1)) and the
    sequence metadata of workload ``w``.  Dense tensors are [B, H, S, D];
    packed tensors are [T, H, D] with int32 ``cu_seqlens_*`` (slot starts,
    B + 1 entries) and ``seq_lens_*`` (valid rows)."""
    if w.layout == "thd":
        qs = (w.total_q, w.heads_q, w.head_dim)
        ks = (w.total_kv, w.heads_kv, w.head_dim)
    else:
        qs = (w.batch, w.heads_q, w.seq_q, w.head_dim)
        ks = (w.batch, w.heads_kv, w.seq_kv, w.head_dim)
    out = dict(
        q=_randn(qs, w.dtype, device, _seed(w, "q", seed)),
        k=_randn(ks, w.dtype, device, _seed(w, "k", seed)),
        v=_randn(ks, w.dtype, device, _seed(w, "v", seed)),
        dO=_randn(qs, w.dtype, device, _seed(w, "dO", seed)),
        sink=None, cu_seqlens_q=None, cu_seqlens_kv=None, seq_lens_q=None, seq_lens_kv=None,
    )
    if w.sink:
        out["sink"] = _randn((w.heads_q,), torch.float32, device, _seed(w, "sink", seed))
    if w.layout == "thd":
        cq = [0]
        for c in w.cap_q:
            cq.append(cq[-1] + c)
        ck = [0]
        for c in w.cap_kv:
            ck.append(ck[-1] + c)
        out["cu_seqlens_q"] = torch.tensor(cq, dtype=torch.int32, device=device)
        out["cu_seqlens_kv"] = torch.tensor(ck, dtype=torch.int32, device=device)
    if w.layout == "thd" or w.pad_len_q or w.pad_len_kv:
        out["seq_lens_q"] = torch.tensor(w.valid_len_q(), dtype=torch.int32, device=device)
        out["seq_lens_kv"] = torch.tensor(w.valid_len_kv(), dtype=torch.int32, device=device)
    return out


def attended_pairs_per_head(w: Workload) -> int:
    """Attended (query, key) pairs of one query head, summed over sequences,
    counted in closed form per row: the key interval of row i is
    [max(0, a - W), min(a + R, s_kv - 1)] with a = i (+ s_kv - s_q if
    bottom-right) and R the right band; this is workload bookkeeping for
    the FLOP count."""
    total = 0
    for lq, lk in zip(w.valid_len_q(), w.valid_len_kv()):
        diag = (lk - lq) if w.bottom_right else 0
        for i in range(lq):
            a = i + diag
            lo = max(0, a - w.window_left) if w.window_left >= 0 else 0
            hi = min(a + w.window_right, lk - 1) if w.causal else lk - 1
            if hi >= lo:
                total += hi - lo + 1
    return total


def flops(w: Workload) -> float:
    """Backward FLOPs on attended pairs: 10 * head_dim per pair per query head
    (five GEMM-shaped products of 2 * head_dim each)."""
    return 10.0 * w.head_dim * attended_pairs_per_head(w) * w.heads_q
