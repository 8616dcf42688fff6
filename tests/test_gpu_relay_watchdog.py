"""The relay watchdog, forced from the host: with the test hook every relay
wait targets a turn that no visitor releases and gives up after a few spins,
so every kernel still runs to its end.  The run must then report
SDPA_ERR_RELAY_TIMEOUT, poison (NaN) the dQ rows of exactly the q-tiles that
had a later turn, and leave every other output bitwise as in a normal run
(the ordered modes are repeatable)."""
import pytest
import torch

from gpu_harness import gpu_backward, gpu_forward, say
from sliding_window_attention_flash_amd import _lib, api
from sliding_window_attention_flash_amd.synth import Workload, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # streaming kernel, chunk relay (boundary q-tiles have two visiting chunks)
    (Workload("wd_stream_b2_h4_s4096_w128", torch.bfloat16, 2, 4, 4, 64, 4096, 4096, window_left=128,
              scale=0.125, engine=2), 1),
    # per-tile kernel, the per-kv-tile relay
    (Workload("wd_tile_gqa_br_w100_d128", torch.bfloat16, 2, 8, 2, 128, 500, 700, bottom_right=True,
              window_left=100), 2),
]


@pytest.mark.parametrize("w,det", CASES, ids=[c[0].name for c in CASES])
def test_forced_relay_timeout_reports_and_poisons(w, det):
    say(f"case {w.name} det={det}: normal run, then every relay wait forced to give up")
    inp = make_inputs(w, device="cuda", seed=31)
    o, lse = gpu_forward(w, inp)
    bw0 = gpu_backward(w, inp, o, lse, deterministic=det)
    dq0, dk0, dv0, _ = (t.clone() if t is not None else None for t in bw0.run())
    torch.cuda.synchronize()
    assert bw0.relay_expiries() == 0

    bw = gpu_backward(w, inp, o, lse, deterministic=det)
    api.sdpa_bwd_plan_set_relay_watchdog(bw.plan, 16, True)
    dq, dk, dv, _ = bw.run()
    torch.cuda.synchronize()
    n = bw.relay_expiries()
    say(f"    expired waits: {n}")
    assert n > 0
    with pytest.raises(_lib.SdpaError) as e:
        api.sdpa_bwd_relay_expiries(bw.plan, bw.workspace, raise_on_timeout=True)
    assert e.value.status == _lib.SDPA_ERR_RELAY_TIMEOUT
    # dK and dV do not go through the relay
    assert torch.equal(dk, dk0) and torch.equal(dv, dv0)
    # dQ: whole q-tiles are NaN, every other row is bitwise the normal run's
    B, H, S, D = dq.shape
    nan_row = torch.isnan(dq).any(dim=-1)                   # [B, H, S]
    assert torch.equal(torch.isnan(dq).all(dim=-1), nan_row), "partly poisoned rows"
    tiles = nan_row.view(B, H, S // 64, 64) if S % 64 == 0 else None
    keep = ~nan_row
    assert torch.equal(dq[keep], dq0[keep]), "rows outside poisoned q-tiles changed"
    if det == 2:
        # per-kv-tile relay: q-tiles with several visiting kv-tiles are
        # poisoned; waits = sum over them of (visitors - 1)
        s = api.sdpa_bwd_schedule(bw.plan, S, w.seq_kv)
        want = torch.zeros(B, H, S, dtype=torch.bool)
        waits = 0
        for i in range(s["n_q"]):
            nv = s["kv_last"][i] - s["kv_first"][i] + 1
            if nv > 1:
                want[:, :, 64 * i:64 * (i + 1)] = True
                waits += (nv - 1) * B * H
        assert torch.equal(nan_row.cpu(), want), "poisoned rows differ from the multi-visitor q-tiles"
        assert n == waits
    else:
        # chunk relay: a boundary q-tile has two visiting chunks, so one wait
        # (turn 1) per poisoned q-tile, and its 64 rows are poisoned together
        full = tiles.all(dim=-1)
        assert torch.equal(tiles.any(dim=-1), full), "q-tile partly poisoned"
        assert int(full.sum()) == n
