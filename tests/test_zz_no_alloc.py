"""sdpa_bwd_run_noalloc (the library's own scratch workspace) against
sdpa_bwd_run (a caller workspace) on the same inputs, through the C ABI:
bitwise in the ordered modes, within the parity bar in the unordered mode.
Calls come in a row on one GPU, each next one smaller, so the scratch holds
the previous call's contents when a call starts."""
import pytest
import torch

from gpu_harness import assert_close, gpu_backward, gpu_forward, say
from sliding_window_attention_flash_amd import api
from sliding_window_attention_flash_amd.synth import Workload, make_inputs

pytestmark = pytest.mark.gpu

BF16, F16 = torch.bfloat16, torch.float16

# largest first: each later call finds the earlier call's data in the scratch
SEQUENCE = [
    (Workload("na_stream_relay_b2_h8_s4096_w128", BF16, 2, 8, 8, 64, 4096, 4096, window_left=128,
              scale=0.125, engine=2), 1),
    (Workload("na_qstream_gqa_br_w96_d128", BF16, 2, 8, 2, 128, 1000, 1064, bottom_right=True, window_left=96,
              engine=5), 1),
    (Workload("na_stream_atomic_b2_h4_s2048_w128", BF16, 2, 4, 4, 64, 2048, 2048, window_left=128,
              scale=0.125, engine=1), 0),
    (Workload("na_tile_relay_gqa_br_w100_d128", BF16, 1, 8, 2, 128, 500, 700, bottom_right=True,
              window_left=100, sink=True), 2),
    (Workload("na_thd_gqa_sink_f16", F16, 3, 4, 2, 64, 192, 256, bottom_right=True, window_left=70, sink=True,
              layout="thd", len_q=(150, 40, 0), len_kv=(256, 100, 30), cap_q=(192, 64, 64),
              cap_kv=(256, 128, 64)), 1),
]


def _run_both(w, det, seed):
    inp = make_inputs(w, device="cuda", seed=seed)
    o, lse = gpu_forward(w, inp)
    ref = gpu_backward(w, inp, o, lse, deterministic=det)
    want = [None if t is None else t.clone() for t in ref.run()]
    bw = gpu_backward(w, inp, o, lse, deterministic=det)  # outputs start as NaN
    assert bw.plan.workspace_bytes <= 64 << 20
    api.sdpa_bwd_run_noalloc(bw.plan, bw.tensors)
    torch.cuda.synchronize()
    got = [bw.dq, bw.dk, bw.dv, bw.dsink]
    return want, got


def test_noalloc_matches_caller_workspace_on_calls_in_a_row():
    for n, (w, det) in enumerate(SEQUENCE):
        say(f"call {n}: {w.name} det={det}")
        want, got = _run_both(w, det, seed=40 + n)
        for name, a, b in zip(("dQ", "dK", "dV", "dSink"), got, want):
            if b is None:
                continue
            assert not torch.isnan(a).any(), f"{name}: NaN (unwritten element?)"
            if det:
                assert torch.equal(a, b), f"{name} differs from sdpa_bwd_run"
            else:
                assert_close(name, a.double().cpu(), b.double().cpu())
