"""GPU parity of the forward kernels (O and LSE) against the fp64 oracle's
forward, element by element, on the same seeded inputs.

The q-major forward (engine 5 on the forward plan: head_dim 128, causal,
W <= 96, dense sequences, diag a multiple of 32, groups of a multiple of 8
query heads) is run forced on its whole domain's corners: both anchors,
windows 0 to 96 (one to four ring tiles), ragged lengths, a single partial
q-step, top-left with fewer keys than queries (rows that see nothing), sink
logits, both 16-bit types, chunks of one q-step and chunks long enough that
the 8-slot ring wraps.  The per-tile forward (engine 3) runs the same shapes.
Outputs start as NaN, so an element no kernel writes fails.
"""
import pytest
import torch

from gpu_harness import _lse_to_gpu_layout, assert_close, mask_kw, oracle_problem, say, seq_kw
from oracle import forward as oracle_forward
from sliding_window_attention_flash_amd import api
from sliding_window_attention_flash_amd.synth import Workload, make_inputs

pytestmark = pytest.mark.gpu

BF16, F16 = torch.bfloat16, torch.float16


def _wl(name, dtype, B, Hq, Hkv, Sq, Skv, **kw):
    return Workload(name, dtype, B, Hq, Hkv, 128, Sq, Skv, **kw)


FWD_QS_CASES = [
    _wl("fq_g8_br_w96_s700", BF16, 1, 8, 1, 700, 700, bottom_right=True, window_left=96),
    _wl("fq_g8_tl_w0_s300", BF16, 2, 16, 2, 300, 300, window_left=0),
    _wl("fq_g8_tl_w1_s97", F16, 1, 8, 1, 97, 97, window_left=1),
    _wl("fq_g8_br_w31_s257x321", BF16, 1, 8, 1, 257, 321, bottom_right=True, window_left=31),
    _wl("fq_g8_tl_w32_s450x700", BF16, 1, 16, 2, 450, 700, window_left=32),
    _wl("fq_g8_br_w33_s1000x1096_f16", F16, 2, 16, 2, 1000, 1096, bottom_right=True, window_left=33),
    _wl("fq_g8_tl_w64_s200", BF16, 1, 8, 1, 200, 200, window_left=64),
    _wl("fq_g8_br_w65_s513", BF16, 1, 8, 1, 513, 513, bottom_right=True, window_left=65),
    # groups of 16 (two heads per wave), 24 (three)
    _wl("fq_g16_br_w96_s640x704", BF16, 2, 32, 2, 640, 704, bottom_right=True, window_left=96),
    _wl("fq_g24_tl_w50_s333", F16, 1, 24, 1, 333, 333, window_left=50),
    # one partial q-step; one row; top-left with fewer keys than queries
    _wl("fq_g8_br_w96_s20x52", BF16, 1, 8, 1, 20, 52, bottom_right=True, window_left=96),
    _wl("fq_g8_tl_w96_s1", BF16, 1, 8, 1, 1, 1, window_left=96),
    _wl("fq_g8_tl_w50_s300x100", BF16, 1, 8, 1, 300, 100, window_left=50),
    # sink logits (the per-tile forward's start values of max and denominator)
    _wl("fq_g8_br_w96_s700x764_sink", BF16, 2, 16, 2, 700, 764, bottom_right=True, window_left=96, sink=True),
    _wl("fq_g16_tl_w40_s300_sink_f16", F16, 1, 16, 1, 300, 300, window_left=40, sink=True),
    _wl("fq_g8_tl_w50_s300x100_sink", F16, 1, 8, 1, 300, 100, window_left=50, sink=True),
    # 64 (sequence, kv head) pairs: chunks of 8 q-steps, so the ring wraps
    _wl("fq_g8_br_w96_b4_h128x16_s1024", BF16, 4, 128, 16, 1024, 1024, bottom_right=True, window_left=96),
]


def _run_forward(w, inp, engine):
    q = inp["q"]
    o = torch.full_like(q, float("nan"))
    lse = torch.full((w.batch, w.heads_q, w.seq_q), float("nan"), dtype=torch.float32, device=q.device)
    fw = api.Forward(q, inp["k"], inp["v"], sink=inp["sink"], engine=engine, o=o, lse=lse,
                     **mask_kw(w), **seq_kw(w, inp))
    fw.run()
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _compare(w, o, lse, ref_o, ref_lse):
    assert not torch.isnan(o).any(), "O: NaN (unwritten element?)"
    assert not torch.isnan(lse).any(), "LSE: NaN (unwritten element?)"
    assert_close("O", o.double(), ref_o)
    lse_r = _lse_to_gpu_layout(w, ref_lse)
    valid = torch.isfinite(lse_r)
    assert torch.equal(torch.isfinite(lse), valid), "LSE: -inf pattern differs"
    err = float((lse.double()[valid] - lse_r[valid]).abs().max()) if valid.any() else 0.0
    say(f"    LSE    max_abs={err:.2e}")
    assert err <= 1e-3, f"LSE max-abs error {err}"


@pytest.mark.parametrize("w", FWD_QS_CASES, ids=[w.name for w in FWD_QS_CASES])
def test_qmajor_forward_full_oracle(w):
    inp = make_inputs(w, device="cuda", seed=13)
    inp_cpu = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    ref_o, ref_lse = oracle_forward(oracle_problem(w), inp_cpu["q"], inp_cpu["k"], inp_cpu["v"], inp_cpu["sink"])
    for engine in (5, 3):
        say(f"case {w.name} forward engine={engine}")
        o, lse = _run_forward(w, inp, engine)
        _compare(w, o, lse, ref_o, ref_lse)


def _forward_random_cases(n=16, seed=4049):
    """Seeded shapes across the q-major forward's domain: groups of 8, 16
    and 24 heads, 1 to 3 kv heads, both anchors (bottom-right offsets that
    are multiples of 32; top-left with more or fewer keys than queries),
    windows 0 to 96, 1 to 1000 query rows, both 16-bit types, with and
    without a sink."""
    import random
    rng = random.Random(seed)
    out = []
    for k in range(n):
        g = rng.choice([8, 8, 16, 24])
        hkv = rng.choice([1, 2, 3])
        b = rng.choice([1, 2])
        sq = rng.choice([1, 31, 32, 33, 95, 160, 257, 511, 1000])
        br = rng.random() < 0.5
        skv = sq + 32 * rng.randint(0, 3) if br else max(1, sq + rng.choice([0, 0, 7, 64, -20]))
        wl = rng.choice([0, 1, 17, 31, 32, 33, 64, 65, 95, 96])
        dt = rng.choice([BF16, F16])
        sink = rng.random() < 0.3
        out.append(_wl(f"fqr{k}_g{g}x{hkv}_b{b}_q{sq}_kv{skv}_{'br' if br else 'tl'}_w{wl}{'_sink' if sink else ''}",
                       dt, b, g * hkv, hkv, sq, skv, bottom_right=br, window_left=wl, sink=sink))
    return out


FWD_RANDOM = _forward_random_cases()


@pytest.mark.parametrize("w", FWD_RANDOM, ids=[w.name for w in FWD_RANDOM])
def test_qmajor_forward_seeded_shapes_full_oracle(w):
    inp = make_inputs(w, device="cuda", seed=7)
    inp_cpu = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    ref_o, ref_lse = oracle_forward(oracle_problem(w), inp_cpu["q"], inp_cpu["k"], inp_cpu["v"], inp_cpu["sink"])
    say(f"case {w.name} forward engine=5")
    o, lse = _run_forward(w, inp, 5)
    _compare(w, o, lse, ref_o, ref_lse)


def test_qmajor_forward_bitwise_repeatable():
    # each (q-step, head) is summed inside one wave in a fixed order
    w = FWD_QS_CASES[0]
    inp = make_inputs(w, device="cuda", seed=31)
    say(f"case {w.name} forward engine=5: 3 runs")
    runs = [_run_forward(w, inp, 5) for _ in range(3)]
    for o, lse in runs[1:]:
        assert torch.equal(o, runs[0][0]) and torch.equal(lse, runs[0][1])
