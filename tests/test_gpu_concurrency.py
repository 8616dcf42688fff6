"""One plan, two streams: concurrent backward runs with distinct workspaces
and outputs give the results of a run alone.

A plan is an immutable host object and a run keeps all of its state
(tickets, relay counters, accumulators) in its own workspace, so runs on
different streams may overlap.  Each case runs the plan eagerly on the
current stream, then issues several interleaved runs on two side streams
(default priority) into two sets of outputs and workspaces, and checks both
against the eager run: bitwise where the dQ path is ordered, within the
parity tolerance where fp32 atomics decide the order of additions.
"""
import ctypes

import pytest
import torch

from gpu_harness import assert_close, gpu_backward, gpu_forward, say
from sliding_window_attention_flash_amd import api
from sliding_window_attention_flash_amd.synth import Workload, make_inputs

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16

CASES = [
    # streaming kernel (forced): chunk relay (ordered) and chunk-boundary atomics
    (Workload("conc_stream_w128_s1500", BF16, 2, 4, 4, 64, 1500, 1500, window_left=128, engine=2), 1),
    (Workload("conc_stream_w128_s1500", BF16, 2, 4, 4, 64, 1500, 1500, window_left=128, engine=1), 0),
    # per-tile path: q-major dQ pass, and the per-kv-tile relay
    (Workload("conc_gqa_br_w90_d128_sink", BF16, 2, 8, 2, 128, 300, 420, bottom_right=True, window_left=90,
              sink=True), 1),
    (Workload("conc_gqa_br_w90_d128_sink", BF16, 2, 8, 2, 128, 300, 420, bottom_right=True, window_left=90,
              sink=True), 2),
]


def _outputs_like(bw):
    dq, dk, dv = torch.empty_like(bw.dq), torch.empty_like(bw.dk), torch.empty_like(bw.dv)
    dsink = torch.empty_like(bw.dsink) if bw.dsink is not None else None
    ws = torch.empty_like(bw.workspace)
    t = api.BwdTensors()
    ctypes.memmove(ctypes.byref(t), ctypes.byref(bw.tensors), ctypes.sizeof(t))
    t.dq, t.dk, t.dv = dq.data_ptr(), dk.data_ptr(), dv.data_ptr()
    t.dsink = dsink.data_ptr() if dsink is not None else None
    return (dq, dk, dv, dsink), t, ws


@pytest.mark.parametrize("w,det", CASES, ids=[f"{w.name}-det{d}" for w, d in CASES])
def test_concurrent_runs_of_one_plan(w, det):
    say(f"case {w.name} det={det}: eager run, then 4 interleaved runs on two streams")
    inp = make_inputs(w, device="cuda", seed=41)
    o, lse = gpu_forward(w, inp)
    bw = gpu_backward(w, inp, o, lse, deterministic=det)
    ref = [t.clone() if t is not None else None for t in bw.run()]
    torch.cuda.synchronize()
    sets = [_outputs_like(bw) for _ in range(2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(4):
        for (outs, t, ws), s in zip(sets, streams):
            with torch.cuda.stream(s):
                for x in outs:
                    if x is not None:
                        x.fill_(float("nan"))
                api.sdpa_bwd_run(bw.plan, t, ws, s)
    torch.cuda.synchronize()
    ordered = det != 0 or api.sdpa_bwd_schedule(bw.plan, 1, 1)["tile_kv"] != 128
    for n, (outs, _, ws) in enumerate(sets):
        for name, got, want in zip(("dq", "dk", "dv", "dsink"), outs, ref):
            if want is None:
                continue
            if ordered:
                assert torch.equal(got, want), f"stream {n}: {name} differs from the run alone"
            else:
                assert_close(f"stream {n} {name}", got.float().cpu(), want.double().cpu())
        if det:
            assert api.sdpa_bwd_relay_expiries(bw.plan, ws) == 0
