"""Pins for the oracle's Chunk-Aware Growth schedule and block budget.

CAG (Light Forcing summary, execution flow, stage 1; gist.science technical summary,
section 2.1): chunk 1 dense, s_i = s_base - alpha_i * beta for i > 1, beta fixed by the
total-FLOP target. The oracle finds beta as the root of the affine FLOP constraint from
two evaluations; the pins below use an independent hand-derived closed form, the
constraint itself as an invariant, and special cases.
"""
import math

import numpy as np
import pytest

import oracle


def _closed_form_beta(F, alpha, s_base, s_t):
    # Hand derivation: sum_{i>=2} F_i (s_base - alpha_i beta) = s_t * sum_i F_i
    #   => beta = (s_base * sum_{i>=2} F_i - s_t * sum_i F_i) / sum_{i>=2} F_i alpha_i
    num = s_base * sum(F[1:]) - s_t * sum(F)
    den = sum(f * a for f, a in zip(F[1:], alpha[1:]))
    return num / den


@pytest.mark.parametrize("s_t", [0.80, 0.85, 0.70, 0.90])
def test_beta_matches_hand_closed_form(s_t):
    F = [float(i) for i in range(1, 8)]              # 7 chunks of 3 frames: F_i ~ i
    alpha = [1.0 / math.sqrt(4 * i) for i in range(1, 8)]
    s, beta = oracle.cag_schedule(7, 4, 0.95, s_t, F)
    assert beta == pytest.approx(_closed_form_beta(F, alpha, 0.95, s_t), rel=1e-13, abs=1e-15)
    for i in range(2, 8):
        assert s[i - 1] == pytest.approx(0.95 - alpha[i - 1] * beta, abs=1e-15)


def test_seven_chunk_values_by_hand():
    # sum_{i=2..7} i * alpha_i = sum sqrt(i)/2 with alpha_i = 1/(2 sqrt(i)) at T = 4.
    half_root_sum = sum(math.sqrt(i) for i in range(2, 8)) / 2
    s, beta = oracle.cag_schedule(7, 4, 0.95, 0.80, list(range(1, 8)))
    assert beta == pytest.approx((0.95 * 27 - 0.80 * 28) / half_root_sum, rel=1e-13)
    assert beta == pytest.approx(0.520935, abs=5e-7)
    assert s[6] == pytest.approx(0.851553, abs=5e-7)
    s, beta = oracle.cag_schedule(7, 4, 0.95, 0.85, list(range(1, 8)))
    assert beta == pytest.approx(0.296532, abs=5e-7)
    assert s[6] == pytest.approx(0.893961, abs=5e-7)


@pytest.mark.parametrize("n,T,s_t", [(7, 4, 0.8), (7, 4, 0.85), (5, 2, 0.6), (12, 8, 0.75), (2, 4, 0.4)])
def test_flop_constraint_and_shape(n, T, s_t):
    rng = np.random.default_rng(n * 100 + T)
    F = rng.uniform(0.5, 3.0, size=n).cumsum()
    s, beta = oracle.cag_schedule(n, T, 0.95, s_t, F)
    assert s[0] == 0.0                                       # chunk 1 dense
    assert float(np.dot(F, s)) == pytest.approx(s_t * F.sum(), rel=1e-12)
    assert beta >= 0
    assert np.all(s[1:] <= 0.95 + 1e-15)
    assert np.all(np.diff(s) >= -1e-15)                      # non-decreasing growth
    assert np.all((s >= 0) & (s < 1))


def test_uniform_alpha_gives_uniform_allocation():
    # alpha_i constant for i > 1: every sparse chunk gets the same s, which the
    # constraint fixes to s_t * sum F / sum_{i>=2} F (the uniform-allocation baseline).
    F = [1.0, 2.0, 3.0, 4.0]
    s, _ = oracle.cag_schedule(4, 4, 0.95, 0.6, F, alpha=[0.3] * 4)
    expect = 0.6 * sum(F) / sum(F[1:])
    assert np.allclose(s[1:], expect, atol=1e-14)


@pytest.mark.parametrize("s_t", [0.93, 0.2])
def test_infeasible_targets_raise(s_t):
    # 0.93 > 0.95*27/28 needs beta < 0; 0.2 drives s_2 below zero.
    with pytest.raises(ValueError):
        oracle.cag_schedule(7, 4, 0.95, s_t, list(range(1, 8)))


def test_block_budget_rule_and_sweep_table():
    # Budget of the 30-layer sweep (target 0.85): W_f = 1 sink + 3 current + min(4, |M|).
    s, _ = oracle.cag_schedule(7, 4, 0.95, 0.85, list(range(1, 8)))
    kb = []
    for i in range(1, 8):
        n_mem = max(0, 3 * i - 4)
        W_f = (3 if i == 1 else 4) + min(4, n_mem)
        kb.append(oracle.block_budget(s[i - 1], 25 * 3 * i, W_f, 25))
    assert kb == [25, 4, 4, 5, 5, 6, 7]
    # realised block-pair density of the schedule: 75 query blocks per chunk and head
    W_b = [3 * 25, 6 * 4, 8 * 4, 8 * 5, 8 * 5, 8 * 6, 8 * 7]
    dense_pairs = sum(75 * 75 * i for i in range(1, 8))
    assert sum(75 * w for w in W_b) / dense_pairs == pytest.approx(0.15, abs=1e-12)
    # round half up, clamps
    assert oracle.block_budget(0.5, 10, 2, 25) == 3          # x = 2.5 -> 3
    assert oracle.block_budget(0.99, 10, 8, 25) == 1         # clamp low
    assert oracle.block_budget(0.0, 500, 2, 25) == 25        # clamp high


def test_uniform_schedule_pins():
    """The uniform allocation: a worked case by hand, the budget identity, and agreement
    with the CAG solver at a constant alpha (where CAG's growth term vanishes)."""
    # F = (1, 2), target 0.5: keep 1.5 = 1 + 2 (1 - s')  ->  s' = 0.75
    assert np.allclose(oracle.uniform_schedule(2, 0.5, [1.0, 2.0]), [0.0, 0.75], rtol=0, atol=1e-15)
    rng = np.random.default_rng(3)
    for n in (3, 7, 12):
        F = rng.uniform(0.5, 2.0, n).cumsum()
        for st in (0.3, 0.6, 0.8):
            s = oracle.uniform_schedule(n, st, F)
            assert s[0] == 0.0 and np.ptp(s[1:]) == 0.0
            assert abs(np.dot(F, 1 - s) - (1 - st) * F.sum()) < 1e-12 * F.sum()
            s_c, beta = oracle.cag_schedule(n, 4, 0.99, st, F, alpha=np.ones(n))
            assert np.allclose(s_c, s, rtol=0, atol=1e-12) and beta >= 0
    with pytest.raises(ValueError):
        oracle.uniform_schedule(3, 0.95, [1.0, 1.0, 1.0])     # s' = 1.425
