"""The backward and forward captured into a HIP graph replay correctly.

Every piece of per-run state (relay counters, the tile ticket, the dQ
accumulator tiles) is reset by a kernel of the run itself, so a captured
run holds kernel nodes only.  Each replay here follows eager work that
overwrites the outputs and a synchronization, and is checked against the
eager result: bitwise where the path is deterministic (the ordered relay,
and the unordered general path, whose dQ pass has no atomics), within the
parity tolerance where fp32 atomics decide the order of additions.
"""
import pytest
import torch

from gpu_harness import assert_close, gpu_backward, gpu_forward, say
from sliding_window_attention_flash_amd import api
from sliding_window_attention_flash_amd.synth import Workload, make_inputs

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16

CASES = [
    # multi-head, causal, window 128, head_dim 64: the streaming kernel
    # (forced: its chunk relay, then its chunk-boundary atomics)
    (Workload("graph_stream_w128_s1000", BF16, 1, 4, 4, 64, 1000, 1000, window_left=128, engine=2), True),
    (Workload("graph_stream_w128_s1000", BF16, 1, 4, 4, 64, 1000, 1000, window_left=128, engine=1), False),
    # GQA, bottom-right, sinks: the per-tile kernel (relay) or the split dQ pass
    (Workload("graph_gqa_br_w70_sink", BF16, 2, 8, 2, 64, 190, 230, bottom_right=True, window_left=70,
              sink=True), 2),
    (Workload("graph_gqa_br_w70_sink", BF16, 2, 8, 2, 64, 190, 230, bottom_right=True, window_left=70,
              sink=True), 0),
    # head_dim 128, groups of 8, W = 96: the q-major streaming kernel (its
    # chunk-boundary fix pass included), after the q-major forward
    (Workload("graph_qstream_g8_br_w96_sink", BF16, 1, 16, 2, 128, 700, 764, bottom_right=True, window_left=96,
              sink=True, engine=5), 1),
]

# the per-tile forward, and the q-major forward (head_dim 128, groups of 8)
FWD_CASES = [CASES[2][0], CASES[4][0]]


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("w,det", CASES, ids=[f"{w.name}-det{int(d)}" for w, d in CASES])
def test_backward_graph_replays_match_eager(w, det):
    say(f"case {w.name} det={det}: eager, capture, 4 replays")
    inp = make_inputs(w, device="cuda", seed=31)
    o, lse = gpu_forward(w, inp)
    bw = gpu_backward(w, inp, o, lse, deterministic=det)
    outs = [t for t in bw.run() if t is not None]
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    exact = det or w.engine != 1  # only the fp32 atomics depend on timing
    g = _capture(bw.run)
    for rep in range(4):
        for t in outs:
            t.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("dq", "dk", "dv", "dsink"), outs, eager):
            if exact:
                assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager run"
            else:
                assert_close(f"replay {rep} {name}", got.float().cpu(), want.double().cpu())
        if det:
            assert bw.relay_expiries() == 0


@pytest.mark.parametrize("w", FWD_CASES, ids=[w.name for w in FWD_CASES])
def test_forward_graph_replays_match_eager(w):
    say(f"case {w.name}: forward, eager, capture, 3 replays")
    inp = make_inputs(w, device="cuda", seed=32)
    fw = api.Forward(inp["q"], inp["k"], inp["v"], sink=inp["sink"], causal=w.causal,
                     bottom_right=w.bottom_right, window_left=w.window_left, scale=w.softmax_scale)
    o, lse = fw.run()
    torch.cuda.synchronize()
    eo, el = o.clone(), lse.clone()
    g = _capture(fw.run)
    for rep in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, eo) and torch.equal(lse, el), f"forward replay {rep} differs"
