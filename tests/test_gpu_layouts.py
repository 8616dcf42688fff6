"""GPU: tensors held sequence-major ([B, S, H, D] memory, passed as the
[B, H, S, D] view most callers have) give the results of contiguous
[B, H, S, D] tensors: the forward and the ordered dQ modes bit for bit, the
unordered mode within the parity tolerance.  Covers the three main kernels
and row strides of H * D elements."""
import pytest
import torch

from gpu_harness import assert_close, gpu_backward, gpu_forward, say, stream_engine
from sliding_window_attention_flash_amd.synth import Workload

pytestmark = pytest.mark.gpu

CASES = [
    # multi-head, causal, window 128, head_dim 64: the streaming kernel
    Workload("seqmajor_stream_tl_w128", torch.bfloat16, 2, 4, 4, 64, 700, 700, window_left=128),
    # GQA, bottom-right, head_dim 128, sinks: the per-tile path
    Workload("seqmajor_gqa_br_w80_d128_sink", torch.float16, 2, 8, 2, 128, 300, 420, bottom_right=True,
             window_left=80, sink=True),
    # GQA, bottom-right, head_dim 128, window 96: the q-major streaming
    # kernel in the unordered and ordered modes (the plan's choice)
    Workload("seqmajor_qstream_gqa_br_w96_d128", torch.bfloat16, 2, 8, 2, 128, 700, 700, bottom_right=True,
             window_left=96),
    # groups of 8: the q-major forward too, on sequence-major strides
    Workload("seqmajor_qstream_g8_br_w96_d128", torch.bfloat16, 1, 16, 2, 128, 700, 764, bottom_right=True,
             window_left=96),
]


def _seq_major(t: torch.Tensor) -> torch.Tensor:
    """The same values, stored [B, S, H, D]."""
    return t.transpose(1, 2).contiguous().transpose(1, 2)


@pytest.mark.parametrize("det", [0, 1, 2], ids=["unordered", "ordered", "tile_relay"])
@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_sequence_major_matches_contiguous(w, det):
    from sliding_window_attention_flash_amd.synth import make_inputs

    say(f"case {w.name} det={det}: sequence-major against contiguous")
    inp = make_inputs(w, device="cuda", seed=13)
    o, lse = gpu_forward(w, inp)
    eng = stream_engine(w, det)  # the streaming kernel where it applies
    ref = [None if t is None else t.clone()
           for t in gpu_backward(w, inp, o, lse, deterministic=det, engine=eng).run()]

    sinp = dict(inp)
    for key in ("q", "k", "v", "dO"):
        sinp[key] = _seq_major(inp[key])
    assert sinp["q"].stride(2) == w.heads_q * w.head_dim and sinp["k"].stride(2) == w.heads_kv * w.head_dim
    so, slse = gpu_forward(w, sinp)
    assert so.stride() == sinp["q"].stride()
    assert torch.equal(so, o) and torch.equal(slse, lse)
    out = gpu_backward(w, sinp, so, slse, deterministic=det, engine=eng).run()
    assert out[0].stride() == sinp["q"].stride() and out[1].stride() == sinp["k"].stride()
    for name, got, want in zip(("dq", "dk", "dv", "dsink"), out, ref):
        if want is None:
            continue
        if det:
            assert torch.equal(got, want), name
        else:
            assert_close(name, got.float().cpu(), want.double().cpu())
