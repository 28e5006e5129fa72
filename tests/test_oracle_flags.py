"""Pins for the oracle's residual-draw flag, its empty-support draw and its
input-error reading (CPU only).

A chain is flagged when a perturbation of at most eps = 1e-6 in any
log-probability difference ln q(v) - ln p(v) or in any perturbed score could
change its emitted token (the north star's "within 1e-6 of its threshold",
read for a draw). The rows below are built so that the answer is known by
construction, and the flag is also checked against a brute-force search: the
draw is re-run on every corner perturbation of the three ids' differences and
scores, and the token must change under one of them exactly when the chain is
flagged.

The residual is max(p - q, 0) (Speculative Speculative Decoding, technical
summary section 2, optimisation 2; SpecTr-GBV section 2, termination step).
An empty support -- p <= q everywhere, possible only through rounding since
both sum to one -- is drawn from p_n with the same noise.
"""
import itertools

import numpy as np
import pytest
from scipy.special import log_softmax

import oracle
from oracle import specverify as sv

EPS = sv.FLAG_EPS
SEED = 0xC0FFEE
POS = 8   # G_1 - G_2 = 2.37 at this position: the constructions below need G_1 > G_2


def _noise(V=3):
    return sv.sampling_noise(SEED, np.array([0]), np.array([POS]), V)[0]


def _residual_case(zt0, zd0):
    """gamma = 1, V = 3, T = 1: target row 0 gives id 0 no mass, the draft token is id 0,
    so position 0 always rejects and the token is the residual draw of row 0."""
    zt = np.stack([zt0, np.zeros(3)])[None]
    zd = np.asarray(zd0, dtype=np.float64)[None, None, None]
    return oracle.verify(zt, zd, np.array([[[0]]]), np.ones(1, np.float32), SEED, np.array([POS]))


def _brute_force_fragile(zt0, zd0):
    """True when some corner perturbation (each ln q(v) - ln p(v) by -eps, 0 or +eps, each
    score by -eps, 0 or +eps) changes the residual draw of the row pair."""
    lp = log_softmax(np.asarray(zt0, dtype=np.float64))
    lq = log_softmax(np.asarray(zd0, dtype=np.float64))
    G = _noise()
    base = np.argmax(sv.residual_log_weights(lp, lq) + G)
    for dq in itertools.product((-EPS, 0.0, EPS), repeat=3):
        w = sv.residual_log_weights(lp, lq + np.array(dq))
        for ds in itertools.product((-EPS, 0.0, EPS), repeat=3):
            if np.argmax(w + G + np.array(ds)) != base:
                return True
    return False


def _support_flip_rows(delta, gap=1.0):
    """Id 1 at ln q - ln p = -delta (in the support, tiny residual) winning by `gap` over
    id 2; for delta < eps a perturbation removes id 1 from the support."""
    G = _noise()
    A = 0.3
    p1, p2 = np.exp(A) / (np.exp(A) + 1), 1 / (np.exp(A) + 1)
    r1 = p1 * -np.expm1(-delta)
    r2 = r1 * np.exp(G[1] - G[2] - gap)
    q1, q2 = p1 * np.exp(-delta), p2 - r2
    q0 = 1.0 - q1 - q2
    return np.array([-np.inf, A, 0.0]), np.log([q0, q1, q2])


def _support_entry_rows(delta, gap=1.0):
    """Id 1 at ln q - ln p = +delta (outside the support); if it entered with the residual
    it would have at d = -(eps - delta) it would win by `gap` over id 2, the only id in the
    support."""
    G = _noise()
    A = 0.3
    p1, p2 = np.exp(A) / (np.exp(A) + 1), 1 / (np.exp(A) + 1)
    w1 = p1 * abs(EPS - delta)
    r2 = w1 * np.exp(G[1] - G[2] - gap)
    q1 = p1 * np.exp(delta)
    q0 = r2 - (q1 - p1)                  # so that p2 - q2 = r2
    q2 = 1.0 - q0 - q1
    assert q0 > 0 and q2 > 0
    return np.array([-np.inf, A, 0.0]), np.log([q0, q1, q2])


def _near_tie_rows(gap):
    """Ids 1 and 2 both at q = p / 2 (deep inside the support); their scores
    ln r + G differ by `gap` (id 1 ahead when gap > 0)."""
    G = _noise()
    A = gap - (G[1] - G[2])
    p = np.exp(log_softmax(np.array([-np.inf, A, 0.0])))
    return np.array([-np.inf, A, 0.0]), np.log([0.5, p[1] / 2, p[2] / 2])


@pytest.mark.parametrize("delta,flagged", [(5e-7, True), (2e-7, True), (1e-5, False),
                                           (3e-5, False)])
def test_support_flip_of_the_winner_is_flagged_within_eps(delta, flagged):
    zt0, zd0 = _support_flip_rows(delta)
    out = _residual_case(zt0, zd0)
    assert out["accept_len"][0, 0] == 0
    assert out["out_token"][0, 0] == 1
    assert bool(out["flagged"][0, 0]) == flagged
    assert _brute_force_fragile(zt0, zd0) == flagged


@pytest.mark.parametrize("delta,flagged", [(5e-7, True), (1e-5, False)])
def test_support_entry_of_a_runner_up_is_flagged_within_eps(delta, flagged):
    zt0, zd0 = _support_entry_rows(delta)
    out = _residual_case(zt0, zd0)
    assert out["accept_len"][0, 0] == 0
    assert out["out_token"][0, 0] == 2
    assert bool(out["flagged"][0, 0]) == flagged
    assert _brute_force_fragile(zt0, zd0) == flagged


@pytest.mark.parametrize("gap,flagged", [(3e-6, True), (-3e-6, True), (1e-7, True),
                                         (5e-6, False), (-1e-5, False), (0.5, False)])
def test_score_near_tie_is_flagged_within_eps(gap, flagged):
    # both ids at q = p/2: the bound moves each score by eps (difference) + eps (score),
    # so the winner is fragile exactly when the two scores are within 4 eps
    zt0, zd0 = _near_tie_rows(gap)
    out = _residual_case(zt0, zd0)
    assert out["out_token"][0, 0] == (1 if gap > 0 else 2)
    assert bool(out["flagged"][0, 0]) == flagged
    assert _brute_force_fragile(zt0, zd0) == flagged


def test_empty_support_draws_from_p_with_the_same_noise():
    # Equal target and draft rows: ln q - ln p is exactly 0 for every id, the residual has
    # no support, and the token is the Gumbel-max draw from p_n -- here written out with
    # SciPy's log_softmax: argmax_v ln p(v) + G_v.
    rng = np.random.default_rng(4)
    V, T = 9, np.float32(0.7)
    for trial in range(20):
        zt = rng.normal(0, 2, size=(1, 2, V))
        zd = zt[:, None, :1].copy()
        n = np.zeros((1, 1), dtype=np.int64)
        lnz_t = oracle.normalize_rows(zt, np.full((1, 1), T, np.float64))[0]
        lnz_d = lnz_t[:, :1][:, None, :]
        tok, flag, empty = sv.sample_tokens(zt, zd, np.array([T], np.float64), lnz_t, lnz_d,
                                            np.zeros((1, 2), np.int64), n, SEED + trial,
                                            np.array([POS]), np.array([[0]]))
        G = sv.sampling_noise(SEED + trial, np.array([0]), np.array([POS]), V)[0]
        want = np.argmax(log_softmax(zt[0, 0] / np.float64(T)) + G)
        assert empty[0, 0]
        assert tok[0, 0] == want
        # every id sits at ln q - ln p = 0 < eps: a perturbation could open the support
        assert flag[0, 0]


@pytest.mark.parametrize("where,value", [("target", np.nan), ("target", np.inf),
                                         ("draft", np.nan), ("draft", np.inf),
                                         ("target", -np.inf)])
def test_non_finite_rows_are_input_errors(where, value):
    rng = np.random.default_rng(9)
    B, g, V = 4, 3, 50
    zt = rng.normal(0, 1, size=(B, g + 1, V))
    zd = zt[:, None, :g] + rng.normal(0, 0.5, size=(B, 1, g, V))
    toks = rng.integers(0, V, size=(B, 1, g))
    T = np.array([0.7, 0.7, 0.0, 0.7], np.float32)
    if value == -np.inf:
        zt[1, 2, :] = -np.inf                        # every entry masked
    elif where == "target":
        zt[1, 2, 17] = value                         # one entry among finite ones
    else:
        zd[1, 0, 1, 17] = value
    zd[2, 0, 0, 3] = np.nan                          # a greedy row's draft is never needed
    out = oracle.verify(zt, zd, toks, T, 5, np.zeros(B, np.int64))
    assert out["error"] == sv.ERR_ROW
    assert out["accept_len"][1, 0] == -1 and out["out_token"][1, 0] == -1
    assert np.all(out["accept_len"][[0, 2, 3], 0] >= 0)
    assert out["chain_error"][2, 0] == 0


def test_greedy_row_with_nan_is_an_input_error():
    zt = np.zeros((1, 2, 5))
    zt[0, 1, 2] = np.nan
    out = oracle.verify(zt, np.zeros((1, 1, 1, 5)), np.array([[[0]]]), np.zeros(1, np.float32), 0,
                        np.zeros(1, np.int64))
    assert out["error"] == sv.ERR_ROW and out["accept_len"][0, 0] == -1
