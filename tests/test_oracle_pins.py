"""The fp64 oracle, pinned to facts other than itself (CPU only)."""
import os

import pytest
import torch

import oracle
import oracle_checks as oc
from oracle import Problem


def test_finite_differences(oracle_lib):
    oc.check_finite_differences()


def test_torch_autograd_explicit_mask(oracle_lib):
    oc.check_torch_autograd()


def test_torch_sdpa_causal_and_long_window(oracle_lib):
    oc.check_torch_sdpa_causal()


def test_closed_forms(oracle_lib):
    oc.check_closed_forms()


def test_invariants(oracle_lib):
    oc.check_invariants()


def test_dense_scan_matches_key_interval(oracle_lib):
    oc.check_dense_scan()


def test_sampled_rows_match_full(oracle_lib):
    oc.check_sampled_rows()


def test_16bit_widening_every_finite_pattern(oracle_lib):
    oc.check_widening()


@pytest.mark.parametrize("S,W,per_seq", [(256, 64, 14560), (4096, 128, 520128), (32768, 128, 4218816)])
def test_attended_pairs_closed_form(oracle_lib, S, W, per_seq):
    # top-left causal + inclusive window W: row i sees min(i, W) + 1 keys, so
    # the count is W(W+1)/2 + (W+1) + (S - W - 1)(W + 1) = sum_i (min(i, W) + 1).
    closed = sum(min(i, W) + 1 for i in range(S))
    assert closed == per_seq
    p = Problem.dense(2, 1, 1, S, S, 8, causal=True, window_left=W)
    assert oracle.attended_pairs(p) == 2 * per_seq


def test_attended_pairs_brute_force(oracle_lib):
    g = torch.Generator().manual_seed(3)
    for _ in range(25):
        sq, skv = (int(x) for x in torch.randint(1, 40, (2,), generator=g))
        w = int(torch.randint(-1, 12, (1,), generator=g))
        causal = bool(torch.randint(0, 2, (1,), generator=g))
        br = bool(torch.randint(0, 2, (1,), generator=g))
        wr = int(torch.randint(0, 6, (1,), generator=g)) if causal else 0
        m = oc.explicit_mask(sq, skv, causal, br, w, wr)
        p = Problem.dense(1, 1, 1, sq, skv, 8, causal=causal, bottom_right=br, window_left=w,
                          window_right=wr)
        assert oracle.attended_pairs(p) == int(m.sum())


MUTANTS = {
    1: "dQ without the softmax scale",
    2: "exclusive window (anchor - j < W)",
    3: "dS sign flipped",
    4: "sink missing from the softmax denominator",
    5: "dK built from dO instead of Q",
    6: "bottom-right anchor shifted the wrong way",
    7: "dSink sign flipped",
    8: "GQA head map h % H_kv instead of h / G",
    9: "exclusive right band (j - anchor < R)",
    10: "f16 exponent bias off by one (2^(e - 24))",
    11: "f16 subnormal scale 2^-25 instead of 2^-24",
    12: "bf16 and f16 storage codes swapped",
    13: "bf16 subnormals flushed to zero",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(tmp_path, mutant):
    """Each planted mistake in the oracle must fail at least one pin."""
    path = oracle.build(str(tmp_path / f"libswa_oracle_m{mutant}.so"), mutant=mutant)
    lib = oracle.load(path)
    failed = []
    for check in oc.ALL_CHECKS:
        try:
            check(lib=lib)
        except AssertionError as e:
            failed.append((check.__name__, str(e)[:80]))
    assert failed, f"mutant {mutant} ({MUTANTS[mutant]}) passed every pin"


def test_golden_regression(oracle_lib):
    """Stored fp64 outputs of a small packed problem (written by
    tests/golden/make_golden.py, which calls only the oracle) still match."""
    from golden import make_golden

    path = os.path.join(os.path.dirname(__file__), "golden", "oracle_small.txt")
    stored = make_golden.read(path)
    fresh = make_golden.compute()
    assert stored.keys() == fresh.keys()
    for key in stored:
        torch.testing.assert_close(fresh[key], stored[key], rtol=1e-12, atol=1e-12)
