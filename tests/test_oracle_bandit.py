"""Pins for the oracle's bandit draft selector (CPU only).

UCB1 is pinned to hand-computed selections and to the finite-time regret bound
of Auer, Cesa-Bianchi and Fischer (2002, Theorem 1); the Gamma and Beta samplers
behind Thompson sampling to SciPy's distributions (Kolmogorov-Smirnov at 0.01);
Thompson sampling to its textbook behaviour on Bernoulli arms (it concentrates
on the best arm and its regret stays far below linear).
"""
import math

import numpy as np
import pytest
from scipy import stats

from oracle import bandit as bd


def test_step_reward():
    assert bd.step_reward(np.array([[3], [1], [4], [0]]), 4) == 8 / 16
    assert bd.step_reward(np.array([[-1], [2]]), 2) == 2 / 4   # an errored chain counts 0


def test_ucb1_hand_sequence():
    b = bd.Bandit(3, bd.UCB1)
    picks = []
    rewards = {0: 0.5, 1: 1.0, 2: 0.0}
    for _ in range(5):
        a = b.select()
        picks.append(a)
        b.update(a, rewards[a])
    # every arm once in index order; then t = 3: indices 0.5 + sqrt(2 ln3) = 1.982,
    # 1 + 1.482 = 2.482, 0 + 1.482 -> arm 1; t = 4: arm 0: 0.5 + sqrt(2 ln 4) = 2.165,
    # arm 1: 1 + sqrt(ln 4) = 2.177, arm 2: 1.665 -> arm 1
    assert picks == [0, 1, 2, 1, 1]
    i0 = 0.5 + math.sqrt(2 * math.log(5) / 1)
    i1 = 1.0 + math.sqrt(2 * math.log(5) / 3)
    assert b.select() == (0 if i0 > i1 else 1)


def test_ucb1_ties_go_to_the_lowest_index():
    b = bd.Bandit(4, bd.UCB1)
    for a in range(4):
        assert b.select() == a
        b.update(a, 0.25)
    assert b.select() == 0


def _run(policy, means, T, seed, reward_seed):
    rng = np.random.default_rng(reward_seed)
    b = bd.Bandit(len(means), policy, seed=seed)
    regret, best = 0.0, max(means)
    counts = np.zeros(len(means), int)
    for _ in range(T):
        a = b.select()
        r = float(rng.random() < means[a])
        b.update(a, r)
        regret += best - means[a]
        counts[a] += 1
    return regret, counts


def test_ucb1_regret_within_the_finite_time_bound():
    means = [0.85, 0.6, 0.4]
    T = 1500
    regs = [_run(bd.UCB1, means, T, 0, s)[0] for s in range(6)]
    gaps = [max(means) - m for m in means if m < max(means)]
    bound = sum(8 * math.log(T) / g for g in gaps) + (1 + math.pi ** 2 / 3) * sum(gaps)
    assert np.mean(regs) <= bound
    assert np.mean(regs) < 0.1 * T          # far below linear


def test_gamma_and_beta_samplers_match_scipy():
    for shape in (1.0, 1.7, 6.5, 40.0):
        xs = [bd.gamma_variate(shape, 1234, t, 0, 0) for t in range(1500)]
        assert stats.kstest(xs, stats.gamma(shape).cdf).pvalue > 0.01, shape
    for a, b in ((1.0, 1.0), (3.0, 1.5), (12.0, 30.0)):
        xs = [bd.beta_variate(a, b, 99, t, 1) for t in range(1500)]
        assert stats.kstest(xs, stats.beta(a, b).cdf).pvalue > 0.01, (a, b)


def test_thompson_concentrates_on_the_best_arm():
    means = [0.5, 0.9, 0.6]
    T = 600
    regret, counts = _run(bd.THOMPSON, means, T, 7, 3)
    assert counts[1] > 0.8 * T
    assert regret < 0.1 * T


def test_thompson_is_reproducible_from_the_seed():
    r1 = _run(bd.THOMPSON, [0.3, 0.6], 100, 5, 1)
    r2 = _run(bd.THOMPSON, [0.3, 0.6], 100, 5, 1)
    assert np.array_equal(r1[1], r2[1])
    r3 = _run(bd.THOMPSON, [0.3, 0.6], 100, 6, 1)
    assert r3[0] >= 0
