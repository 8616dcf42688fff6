"""GPU parity: the HIP path against the fp64 oracle on the same seeded inputs.

Every problem is compared element by element with the full oracle: small
problems (several tiles, ragged tails, every mask variant) and the full-size
workloads (the largest GQA one on whole batch entries), which additionally
get a sampled-row comparison.  Outputs start as NaN so an element the
kernels never write fails the test.
"""
import pytest
import torch

from gpu_harness import (assert_close, batch_entries, compare_full, compare_sampled, oracle_full, run_gpu,
                         say, stream_engine)
from sliding_window_attention_flash_amd.synth import CONFIGS, Workload, packed_lengths

pytestmark = pytest.mark.gpu

BF16, F16 = torch.bfloat16, torch.float16


def _wl(name, dtype, B, Hq, Hkv, D, Sq, Skv, **kw):
    return Workload(name, dtype, B, Hq, Hkv, D, Sq, Skv, **kw)


SMALL = [
    _wl("mha_tl_w17_s300_d64", BF16, 2, 4, 4, 64, 300, 300, window_left=17),
    _wl("gqa_br_w100_d128_f16", F16, 2, 8, 2, 128, 200, 333, bottom_right=True, window_left=100),
    _wl("mqa_tl_causal_d64", BF16, 1, 4, 1, 64, 190, 190),
    _wl("w0_tl_d64", BF16, 1, 2, 2, 64, 130, 130, window_left=0),
    _wl("tl_sq_gt_skv_w40", BF16, 1, 2, 2, 64, 260, 130, window_left=40),
    _wl("swa_only_br_w50", F16, 1, 2, 1, 64, 100, 250, causal=False, bottom_right=True, window_left=50),
    _wl("noncausal_full_d128", BF16, 1, 2, 2, 128, 150, 170, causal=False),
    _wl("sink_gqa_tl_w64_d128", BF16, 2, 6, 3, 128, 257, 257, window_left=64, sink=True),
    _wl("padded_bhsd_w33", F16, 2, 4, 2, 64, 200, 230, bottom_right=True, window_left=33,
        pad_len_q=(200, 77), pad_len_kv=(230, 140)),
    # multi-head, causal, window <= 128, head_dim 64: the streaming kernel
    _wl("stream_tl_w128_s1000", BF16, 2, 4, 4, 64, 1000, 1000, window_left=128, scale=0.125),
    _wl("stream_br_w100_s300x700", BF16, 2, 4, 4, 64, 300, 700, bottom_right=True, window_left=100),
    _wl("stream_br_w128_s777_f16", F16, 1, 3, 3, 64, 777, 777, bottom_right=True, window_left=128),
    _wl("stream_padded_w61", F16, 2, 2, 2, 64, 640, 700, bottom_right=True, window_left=61,
        pad_len_q=(640, 333), pad_len_kv=(700, 500)),
    _wl("stream_sink_w96_s1500", BF16, 1, 2, 2, 64, 1500, 1500, window_left=96, sink=True),
    # right-band widening: keys up to anchor + R
    _wl("rband_tl_w40_r24_d64", BF16, 2, 4, 4, 64, 300, 300, window_left=40, window_right=24),
    _wl("rband_gqa_br_w100_r70_d128_sink", BF16, 2, 8, 2, 128, 200, 333, bottom_right=True, window_left=100,
        window_right=70, sink=True),
    _wl("rband_nowin_r64_sq_gt_skv_f16", F16, 1, 4, 2, 64, 260, 190, window_right=64),
    _wl("rband_mha_s2048_w128_r64", BF16, 1, 4, 4, 64, 2048, 2048, window_left=128, window_right=64,
        scale=0.125),
    # narrow window, GQA: the dQ pass walks runs of q-tiles; rows past
    # s_kv + W see no key, so a run ends in q-tiles no kv-tile visits
    _wl("gqa_tl_sq_gt_skv_w40_runs", BF16, 2, 4, 2, 64, 520, 130, window_left=40),
    _wl("gqa_br_w60_d128_runs_f16", F16, 1, 6, 2, 128, 700, 900, bottom_right=True, window_left=60),
    # softmax scales other than 1/sqrt(head_dim) (and not a power of two):
    # the streaming kernel and the per-tile path
    _wl("stream_tl_w64_scale0p3", BF16, 1, 2, 2, 64, 500, 500, window_left=64, scale=0.3),
    _wl("gqa_br_w50_d128_scale0p2_f16", F16, 1, 4, 2, 128, 200, 260, bottom_right=True, window_left=50,
        scale=0.2),
]


# deterministic: 0 unordered, 1 bitwise repeatable (chunk relay in the
# streaming kernel, q-major dQ pass elsewhere), 2 the per-kv-tile relay
DET = dict(argvalues=[0, 1, 2], ids=["unordered", "ordered", "tile_relay"])


@pytest.mark.parametrize("det", **DET)
@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_small_full_oracle(w, det):
    # shapes the streaming kernel applies to run it (these small ones would
    # take the per-tile kernels by the plan's table, which ENGINE_CASES and
    # the other shapes cover)
    say(f"case {w.name} det={det}")
    inp, out, _ = run_gpu(w, seed=3, deterministic=det, engine=stream_engine(w, det))
    assert out["expiries"] == 0
    compare_full(w, inp, out)


# every engine, forced, on shapes the streaming kernel applies to (so all
# four run): 1 streaming + atomics, 2 streaming + chunk relay, 3 per-tile +
# q-major dQ pass, 4 per-tile + per-kv-tile relay
ENGINE_CASES = [
    _wl("eng_mha_tl_w128_s1500", BF16, 2, 4, 4, 64, 1500, 1500, window_left=128, scale=0.125),
    _wl("eng_mha_br_w77_s600x1100_padded_f16", F16, 2, 3, 3, 64, 600, 1100, bottom_right=True, window_left=77,
        pad_len_q=(600, 411), pad_len_kv=(1100, 950), sink=True),
]


@pytest.mark.parametrize("engine", [1, 2, 3, 4])
@pytest.mark.parametrize("w", ENGINE_CASES, ids=[w.name for w in ENGINE_CASES])
def test_forced_engines_full_oracle(w, engine):
    say(f"case {w.name} engine={engine}")
    inp, out, _ = run_gpu(w, seed=17, deterministic=0, engine=engine)
    compare_full(w, inp, out, check_fwd=engine == 1)


# engine 5, the q-major streaming kernel (head_dim 128, causal, W <= 96, dense,
# diag a multiple of 32): GQA and MHA, both anchors, windows from 0
# to 96, ragged lengths, a tail of keys no row sees (top-left, S_kv > S_q),
# and enough 32-row steps that chunks meet (the plan's chunks are at least
# 3 steps long: 9 steps make three chunks of exactly 3)
QSTREAM_CASES = [
    _wl("qs_gqa8_br_w96_s700", BF16, 1, 8, 1, 128, 700, 700, bottom_right=True, window_left=96),
    _wl("qs_mha_tl_w96_s300", BF16, 1, 2, 2, 128, 300, 300, window_left=96),
    _wl("qs_gqa4_br_w64_s1000x1096_f16", F16, 2, 8, 2, 128, 1000, 1096, bottom_right=True, window_left=64),
    _wl("qs_gqa2_tl_w0_s500", BF16, 1, 4, 2, 128, 500, 500, window_left=0),
    _wl("qs_gqa2_tl_w33_s450x700", BF16, 1, 4, 2, 128, 450, 700, window_left=33),
    _wl("qs_mha_br_w96_s2000", BF16, 1, 2, 2, 128, 2000, 2000, bottom_right=True, window_left=96),
    _wl("qs_gqa8_br_w96_s1200x1264_f16", F16, 2, 16, 2, 128, 1200, 1264, bottom_right=True, window_left=96),
    _wl("qs_gqa3_tl_w17_s900", BF16, 3, 6, 2, 128, 900, 900, window_left=17),
    _wl("qs_gqa4_br_w96_s288x352", BF16, 1, 4, 1, 128, 288, 352, bottom_right=True, window_left=96),
    # one partial q-step; two q-steps, the second of one row
    _wl("qs_gqa2_br_w96_s20x52", BF16, 1, 4, 2, 128, 20, 52, bottom_right=True, window_left=96),
    _wl("qs_mha_tl_w50_s33_f16", F16, 2, 3, 3, 128, 33, 33, window_left=50),
    # sink logits: dSink from per-q-step partials
    _wl("qs_gqa4_br_w96_s700x764_sink", BF16, 2, 8, 2, 128, 700, 764, bottom_right=True, window_left=96, sink=True),
    _wl("qs_mha_tl_w40_s300_sink_f16", F16, 1, 3, 3, 128, 300, 300, window_left=40, sink=True),
]


@pytest.mark.parametrize("det", [0, 1])
@pytest.mark.parametrize("w", QSTREAM_CASES, ids=[w.name for w in QSTREAM_CASES])
def test_qstream_engine_full_oracle(w, det):
    say(f"case {w.name} engine=5 det={det}")
    inp, out, _ = run_gpu(w, seed=11, deterministic=det, engine=5)
    assert out["expiries"] == 0
    compare_full(w, inp, out, check_fwd=False)


def _qstream_random_cases(n=24, seed=2026):
    """Seeded shapes across engine 5's domain: groups of 1 to 8 heads, both
    anchors (bottom-right offsets that are multiples of 32), windows 0 to 96,
    1 to 900 query rows (single partial q-steps, chunks of exactly 3,
    several chunks), both 16-bit types, with and without a sink."""
    import random
    rng = random.Random(seed)
    out = []
    for k in range(n):
        g = rng.choice([1, 2, 3, 4, 8])
        hkv = rng.choice([1, 2, 3])
        b = rng.choice([1, 2])
        sq = rng.choice([1, 17, 32, 95, 96, 97, 288, 300, 513, 900])
        br = rng.random() < 0.5
        skv = sq + 32 * rng.randint(0, 4) if br else sq + rng.choice([0, 0, 5, 64])
        wl = rng.choice([0, 1, 31, 32, 33, 63, 64, 65, 95, 96])
        dt = rng.choice([BF16, F16])
        sink = rng.random() < 0.3
        out.append(_wl(f"qsr{k}_g{g}x{hkv}_b{b}_q{sq}_kv{skv}_{'br' if br else 'tl'}_w{wl}{'_sink' if sink else ''}",
                       dt, b, g * hkv, hkv, 128, sq, skv, bottom_right=br, window_left=wl, sink=sink))
    return out


QSTREAM_RANDOM = _qstream_random_cases()


@pytest.mark.parametrize("w", QSTREAM_RANDOM, ids=[w.name for w in QSTREAM_RANDOM])
def test_qstream_engine_seeded_shapes_full_oracle(w):
    say(f"case {w.name} engine=5")
    inp, out, _ = run_gpu(w, seed=5, deterministic=1, engine=5)
    compare_full(w, inp, out, check_fwd=False)


def test_qstream_engine_bitwise_repeatable():
    # every sum in a fixed order: dQ inside one step, dK / dV in registers over
    # the chunk's steps, the two sides of a shared kv-tile added in turn
    w = QSTREAM_CASES[-2]
    say(f"case {w.name} engine=5: 3 runs")
    _, outs, _ = run_gpu(w, seed=29, deterministic=1, runs=3, engine=5)
    for key in ("dq", "dk", "dv"):
        assert torch.equal(outs[0][key], outs[1][key]) and torch.equal(outs[0][key], outs[2][key]), key


def _thd_small(sink=True, dtype=F16, D=64, hkv=2, wr=0):
    # one sequence with no query rows and one with no keys, slots padded
    lq = (70, 0, 130, 5, 64, 600)
    lk = (300, 40, 130, 0, 200, 900)
    cq = (128, 64, 192, 64, 64, 640)
    ck = (300, 64, 150, 16, 200, 901)
    return Workload(f"thd_small_sink{int(sink)}_d{D}_hkv{hkv}_r{wr}", dtype, 6, 8, hkv, D, max(cq), max(ck),
                    bottom_right=True, window_left=90, window_right=wr, sink=sink, layout="thd",
                    len_q=lq, len_kv=lk, cap_q=cq, cap_kv=ck)


@pytest.mark.parametrize("det", **DET)
@pytest.mark.parametrize("D,hkv,wr", [(64, 2, 0), (128, 2, 0), (64, 8, 0), (64, 2, 50)])
def test_thd_padded_with_sinks(det, D, hkv, wr):
    w = _thd_small(D=D, hkv=hkv, wr=wr)
    say(f"case {w.name} det={det}")
    inp, out, _ = run_gpu(w, seed=5, deterministic=det, engine=stream_engine(w, det))
    compare_full(w, inp, out)


def test_c1_tiny_full_oracle():
    w = CONFIGS["c1"]
    for det in (0, 1, 2):
        say(f"case {w.name} det={det}")
        inp, out, _ = run_gpu(w, seed=1, deterministic=det)
        compare_full(w, inp, out)


def test_relay_bitwise_repeatable_and_matches_atomic():
    w = _wl("det_b2_h4_s2048_w128", BF16, 2, 4, 4, 64, 2048, 2048, window_left=128, scale=0.125,
            deterministic=True, engine=2)
    say(f"case {w.name}: 3 chunk-relay runs + 1 atomic run")
    inp, outs, _ = run_gpu(w, seed=9, runs=3)
    for o in outs:
        assert o["expiries"] == 0
    for key in ("dq", "dk", "dv"):
        assert torch.equal(outs[0][key], outs[1][key]) and torch.equal(outs[0][key], outs[2][key]), key
    _, at, _ = run_gpu(w, seed=9, deterministic=False, engine=1)
    for key in ("dq", "dk", "dv"):
        assert_close(f"{key} det/at", outs[0][key].cpu(), at[key].cpu().double())
    compare_full(w, inp, outs[0], check_fwd=False)


@pytest.mark.parametrize("det,sink", [(1, True), (2, True), (1, False)],
                         ids=["ordered", "tile_relay", "ordered_delta_in_dq_pass"])
def test_general_path_bitwise_repeatable(det, sink):
    # GQA, bottom-right, head_dim 128: the per-tile kernel with the q-major
    # dQ pass (1) or the per-kv-tile relay (2); without a sink the dQ pass
    # walks q-tile runs and forms delta itself
    w = _wl(f"det_gqa_br_w100_d128_s777_sink{int(sink)}", BF16, 2, 8, 2, 128, 777, 900, bottom_right=True,
            window_left=100, sink=sink)
    say(f"case {w.name} det={det}: 3 runs + 1 unordered run")
    inp, outs, _ = run_gpu(w, seed=19, deterministic=det, runs=3)
    for o in outs:
        assert o["expiries"] == 0
    keys = ("dq", "dk", "dv", "dsink") if sink else ("dq", "dk", "dv")
    for key in keys:
        assert torch.equal(outs[0][key], outs[1][key]) and torch.equal(outs[0][key], outs[2][key]), key
    _, un, _ = run_gpu(w, seed=19, deterministic=0)
    for key in keys:
        assert_close(f"{key} det/un", outs[0][key].float().cpu(), un[key].double().cpu())
    compare_full(w, inp, outs[0], check_fwd=False)


def test_gqa_equals_group_sum_of_expanded_mha():
    w = _wl("gqa_8x2_br_w70", BF16, 2, 8, 2, 64, 190, 230, bottom_right=True, window_left=70, sink=True)
    say(f"case {w.name}: GQA vs head-expanded MHA on the GPU")
    inp, out, ginp = run_gpu(w, seed=11)
    from gpu_harness import gpu_backward, gpu_forward
    we = w.with_(name=w.name + "_expanded", heads_kv=8)
    einp = dict(ginp)
    einp["k"] = ginp["k"].repeat_interleave(4, dim=1).contiguous()
    einp["v"] = ginp["v"].repeat_interleave(4, dim=1).contiguous()
    o, lse = gpu_forward(we, einp)
    dq, dk, dv, dsink = gpu_backward(we, einp, o, lse).run()
    torch.cuda.synchronize()
    assert_close("dQ", out["dq"].cpu(), dq.cpu().double())
    assert_close("dK", out["dk"].cpu(), dk.view(2, 2, 4, 230, 64).double().sum(2).cpu())
    assert_close("dV", out["dv"].cpu(), dv.view(2, 2, 4, 230, 64).double().sum(2).cpu())
    assert_close("dSink", out["dsink"].cpu(), dsink.cpu().double())


def test_keys_outside_every_window_are_exact_zero():
    # bottom-right, s_q much shorter than s_kv: keys below s_kv - s_q - W are
    # seen by no query; their kv-tiles run zero iterations and store zeros.
    w = _wl("br_far_keys", BF16, 1, 4, 2, 64, 100, 1000, bottom_right=True, window_left=50)
    say(f"case {w.name}")
    inp, out, _ = run_gpu(w, seed=13)
    first = 1000 - 100 - 50
    assert torch.count_nonzero(out["dk"][:, :, :first]) == 0
    assert torch.count_nonzero(out["dv"][:, :, :first]) == 0
    compare_full(w, inp, out, check_fwd=False)


# ---- full-size workloads -----------------------------------------------------
# Every full-size workload is compared element by element with the full
# oracle (c4, too large for one oracle run, on whole batch entries), with the
# sampled row comparison kept as an extra check.


def test_c2_s4096_full_oracle():
    w = CONFIGS["c2_4k"]
    say(f"case {w.name} (full oracle)")
    inp, out, _ = run_gpu(w, seed=21)
    compare_full(w, inp, out)


def test_c2_s8192_full_oracle():
    w = CONFIGS["c2_8k"]
    say(f"case {w.name} (full oracle, then sampled rows)")
    inp, out, _ = run_gpu(w, seed=22)
    compare_full(w, inp, out)
    compare_sampled(w, inp, out)


def test_c3_s32768_relay_bitwise_and_full_oracle_both_modes():
    w = CONFIGS["c3"]
    say(f"case {w.name}: 3 relay runs, full oracle for the relay and the atomic run")
    inp, outs, _ = run_gpu(w, seed=23, runs=3)
    for o in outs:
        assert o["expiries"] == 0
    for key in ("dq", "dk", "dv"):
        assert torch.equal(outs[0][key], outs[1][key]) and torch.equal(outs[0][key], outs[2][key]), key
    ref = oracle_full(w, inp)
    say("  relay run vs oracle")
    compare_full(w, inp, outs[0], ref=ref)
    compare_sampled(w, inp, outs[0])
    _, at, _ = run_gpu(w, seed=23, deterministic=False, engine=1)
    say("  atomic run vs oracle")
    compare_full(w, inp, at, ref=ref)
    for key in ("dq", "dk", "dv"):
        assert_close(f"{key} det/at", outs[0][key].float(), at[key].float())


@pytest.mark.parametrize("engine", [3, 5])
def test_c4_gqa_s16484_whole_batch_entries_full_oracle(engine):
    # both engines that apply: the per-tile kernels with the q-major dQ pass,
    # and the q-major streaming kernel
    w = CONFIGS["c4"].with_(engine=engine)
    say(f"case {w.name} engine={engine}: batch entries 0 and 11 (all 48 heads, all rows) against the full oracle")
    inp, out, _ = run_gpu(w, seed=24, engine=engine)
    ws, inp2, out2 = batch_entries(w, inp, out, [0, w.batch - 1])
    compare_full(ws, inp2, out2, check_fwd=engine == 3)
    # every entry: no element left unwritten
    for name in ("dq", "dk", "dv"):
        assert not torch.isnan(out[name]).any(), f"{name}: NaN somewhere in the full output"
    compare_sampled(w, inp, out, n_q=192, n_kv=96)


def test_nonsquare_class_whole_batch_entries_full_oracle():
    # the pages' non-square class: b12, 40/8 heads, d64, q128 / kv8960,
    # bottom-right, W8000 (every row sees 8001 keys)
    w = CONFIGS["nonsquare"]
    say(f"case {w.name}: batch entries 0 and 11 against the full oracle, in all three dQ modes")
    ref = None
    for det in (0, 1, 2):
        inp, out, _ = run_gpu(w, seed=27, deterministic=det)
        ws, inp2, out2 = batch_entries(w, inp, out, [0, w.batch - 1])
        if ref is None:
            ref = oracle_full(ws, inp2)
        say(f"  det={det}")
        compare_full(ws, inp2, out2, check_fwd=det == 0, ref=ref)
        for name in ("dq", "dk", "dv"):
            assert not torch.isnan(out[name]).any(), f"{name}: NaN somewhere in the full output"


def test_c4_f16_variant_full_oracle():
    w = CONFIGS["c4_f16"]
    say(f"case {w.name} (full oracle)")
    inp, out, _ = run_gpu(w, seed=25)
    compare_full(w, inp, out)


def test_c5_thd_sinks_full_oracle():
    w = CONFIGS["c5"]
    say(f"case {w.name} (full oracle, dSink)")
    inp, out, _ = run_gpu(w, seed=26)
    compare_full(w, inp, out)
