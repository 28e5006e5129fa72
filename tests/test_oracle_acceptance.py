"""Pins for the oracle's acceptance probability and accept-length law (CPU only).

alpha_j = sum_v min(p_j, q_j) is pinned four ways that do not retype it:
closed forms on rows whose softmax is known exactly, the identity
sum min(p, q) = 1 - TV(p, q) with SciPy's softmax, the T -> 0 limit against the
greedy rule, and -- the pin to the method itself -- replicates of the oracle's
full verification step with draft tokens drawn from q, whose accept-length
frequencies must pass a chi-square gate at 0.01 against outcome_law(alpha)
(FlashSpec, section 3: distribution-equivalence gate at 0.01). A planted
mistake (the temperature dropped from alpha) must fail that gate.
"""
import math

import numpy as np
import pytest
from scipy import stats
from scipy.special import softmax

import oracle
from oracle import acceptance as acc

SEED = 0x0DDC_0FFE_E0DD_F00D


def _alpha1(zt_row, zd_row, T):
    """alpha of one target row and one draft row through the oracle's batch API."""
    target = np.stack([zt_row, zt_row])[None]            # [1, 2, V] (row 1 unused)
    draft = np.asarray(zd_row, dtype=np.float64)[None, None, None]   # [1, 1, 1, V]
    return float(oracle.acceptance_probability(target, draft, np.array([T], np.float32))[0, 0, 0])


def test_closed_form_three_ids():
    # p = (1, 2, 3)/6, q = (3, 2, 1)/6 at T = 1: sum min = (1 + 2 + 1)/6 = 2/3
    zt = np.log([1.0, 2.0, 3.0])
    zd = np.log([3.0, 2.0, 1.0])
    assert math.isclose(_alpha1(zt, zd, 1.0), 2.0 / 3.0, rel_tol=1e-14)
    # T = 2: weights sqrt(1, 2, 3) and sqrt(3, 2, 1): (1 + sqrt 2 + 1) / (1 + sqrt 2 + sqrt 3)
    want = (2.0 + math.sqrt(2.0)) / (1.0 + math.sqrt(2.0) + math.sqrt(3.0))
    assert math.isclose(_alpha1(zt, zd, 2.0), want, rel_tol=1e-14)


def test_identical_and_disjoint_rows():
    rng = np.random.default_rng(3)
    z = rng.normal(0, 2, size=50)
    assert math.isclose(_alpha1(z, z, 0.7), 1.0, rel_tol=1e-14)
    a = np.full(6, -np.inf); a[0] = 0.0
    b = np.full(6, -np.inf); b[5] = 1.0
    assert _alpha1(a, b, 1.0) == 0.0
    law = oracle.outcome_law(np.array([[1.0, 1.0, 1.0]]))
    assert np.array_equal(law, [[0.0, 0.0, 0.0, 1.0]])
    law = oracle.outcome_law(np.array([[0.0, 0.3, 0.9]]))
    assert np.array_equal(law, [[1.0, 0.0, 0.0, 0.0]])


def test_total_variation_identity():
    rng = np.random.default_rng(11)
    B, K, g, V = 3, 2, 4, 257
    zt = rng.normal(0, 1.5, size=(B, g + 1, V))
    zd = zt[:, None, :g] + rng.normal(0, 1.0, size=(B, K, g, V))
    T = np.array([0.5, 1.0, 1.7], dtype=np.float32)
    alpha = oracle.acceptance_probability(zt, zd, T)
    T64 = T.astype(np.float64)
    p = softmax(zt[:, :g] / T64[:, None, None], axis=-1)
    q = softmax(zd / T64[:, None, None, None], axis=-1)
    tv = 0.5 * np.abs(p[:, None] - q).sum(axis=-1)
    np.testing.assert_allclose(alpha, 1.0 - tv, rtol=0, atol=1e-13)
    assert np.all((alpha > 0) & (alpha < 1))


def test_stored_logits_decoded_like_the_step():
    rng = np.random.default_rng(5)
    zt = rng.normal(0, 2, size=(2, 3, 40)).astype(np.float32)
    zd = (zt[:, None, :2] + rng.normal(0, 1, size=(2, 1, 2, 40))).astype(np.float32)
    T = np.array([0.9, 1.3], dtype=np.float32)
    a_raw = oracle.acceptance_probability(zt.astype(np.float64), zd.astype(np.float64), T)
    a_f32 = oracle.acceptance_probability(zt, zd, T, dtype="f32")
    np.testing.assert_array_equal(a_raw, a_f32)


def test_greedy_rule_and_low_temperature_limit():
    zt = np.array([[[0.0, 3.0, 3.0, 1.0], [2.0, 0.0, 0.0, 2.0], [0.0, 0.0, 0.0, 0.0]]])
    # draft argmaxes: row 0 -> id 1 (lowest of the tie 1, 2, like the target), row 1 -> id 3
    zd = np.array([[[[1.0, 5.0, 5.0, 0.0], [0.0, 0.0, 0.0, 4.0]]]])
    a = oracle.acceptance_probability(zt, zd, np.array([0.0], np.float32))
    assert np.array_equal(a, [[[1.0, 0.0]]])
    # separated maxima: a small positive temperature approaches the greedy value
    zt2 = np.array([[[0.0, 3.0, 1.0], [2.0, 0.0, 0.5], [0.0, 0.0, 0.0]]])
    zd2 = np.array([[[[1.0, 4.0, 0.0], [0.0, 0.2, 3.0]]]])
    greedy = oracle.acceptance_probability(zt2, zd2, np.array([0.0], np.float32))
    cold = oracle.acceptance_probability(zt2, zd2, np.array([0.01], np.float32))
    np.testing.assert_allclose(cold, greedy, atol=1e-30)
    assert np.array_equal(greedy, [[[1.0, 0.0]]])


def test_invalid_temperature_gives_nan():
    z = np.zeros((1, 2, 3))
    a = oracle.acceptance_probability(z, z[:, None, :1], np.array([-1.0], np.float32))
    assert np.isnan(a).all()


def test_outcome_law_is_a_distribution():
    rng = np.random.default_rng(8)
    alpha = rng.uniform(0, 1, size=(50, 3, 7))
    law = oracle.outcome_law(alpha)
    np.testing.assert_allclose(law.sum(axis=-1), 1.0, atol=1e-14)
    assert np.all(law >= 0)
    # P(n >= 1) is the first position's acceptance probability
    np.testing.assert_allclose(law[..., 1:].sum(axis=-1), alpha[..., 0], atol=1e-14)
    # constant alpha: a geometric law truncated at gamma
    a = 0.6
    law = oracle.outcome_law(np.full((1, 5), a))[0]
    want = [a ** m * (1 - a) for m in range(5)] + [a ** 5]
    np.testing.assert_allclose(law, want, rtol=1e-14)
    assert math.isclose(float(oracle.expected_accept_length(law)),
                        sum(m * w for m, w in enumerate(want)), rel_tol=1e-14)


# --- the pin to the method: replicates of the full verification step ---------

G, V, N = 3, 6, 400_000
T32 = float(np.float32(0.8))


def _rows():
    rng = np.random.default_rng(2024)
    zt = rng.normal(0, 1.2, size=(G + 1, V))
    zd = zt[:G] + rng.normal(0, 0.9, size=(G, V))
    return zt, zd


def _chi2_pvalue(observed, prob, n):
    exp = prob * n
    stat = np.sum((observed - exp) ** 2 / exp)
    return stats.chi2.sf(stat, len(exp) - 1)


@pytest.fixture(scope="module")
def replicate_lengths():
    zt, zd = _rows()
    q = softmax(zd / T32, axis=1)
    rng = np.random.default_rng(99)
    toks = np.stack([rng.choice(V, size=N, p=q[j]) for j in range(G)], axis=1)
    out = oracle.verify(np.broadcast_to(zt, (N, G + 1, V)), np.broadcast_to(zd, (N, 1, G, V)),
                        toks[:, None, :], np.full(N, T32, dtype=np.float32), SEED,
                        np.zeros(N, dtype=np.int64))
    return out["accept_len"][:, 0]


def test_accept_length_frequencies_follow_the_law(replicate_lengths):
    zt, zd = _rows()
    alpha = oracle.acceptance_probability(zt[None], zd[None, None], np.array([T32], np.float32))
    law = oracle.outcome_law(alpha)[0, 0]
    counts = np.bincount(replicate_lengths, minlength=G + 1)
    assert _chi2_pvalue(counts, law, N) >= 0.01
    mean = replicate_lengths.mean()
    sd = np.sqrt(np.sum(law * (np.arange(G + 1) - oracle.expected_accept_length(law)) ** 2) / N)
    assert abs(mean - oracle.expected_accept_length(law)) < 5 * sd


def test_planted_mistake_fails_the_gate(replicate_lengths):
    # alpha computed without the temperature (T = 1 instead of 0.8)
    zt, zd = _rows()
    wrong = acc.acceptance_probability(zt[None], zd[None, None], np.array([1.0], np.float32))
    law = oracle.outcome_law(wrong)[0, 0]
    counts = np.bincount(replicate_lengths, minlength=G + 1)
    assert _chi2_pvalue(counts, law, N) < 1e-6
