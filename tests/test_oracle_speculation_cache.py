"""Pins for the oracle's residual top-F candidates, geometric fan-out and cache lookup (CPU).

Pinned by: hand-computed fan-outs; a residual whose ordering and support are
known in closed form (p proportional to the id, q uniform); a brute-force
Python sort of SciPy-normalised weights; hand cases for greedy ties and the
lookup; and -- the pin to the method -- replicates of the oracle's full step
with q-drawn drafts, whose cache hit rate must match the rate predicted from the
candidates' residual mass and the accept-length law (binomial bound), with the
most frequent emitted token of every outcome equal to its first candidate. A
planted mistake (candidates ranked by p instead of max(p - q, 0)) must fail.
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle
from oracle import speculation_cache as sc


def test_geometric_fanout_hand_cases():
    assert sc.geometric_fanout(2, 7, 0.5).tolist() == [4, 2, 1]
    # exact 10 * (4, 2, 1) / 7 = 5.71, 2.86, 1.43: floors 5, 2, 1; remainders give j=1, j=0
    assert sc.geometric_fanout(2, 10, 0.5).tolist() == [6, 3, 1]
    assert sc.geometric_fanout(3, 8, 1.0).tolist() == [2, 2, 2, 2]
    assert sc.geometric_fanout(3, 6, 1.0).tolist() == [2, 2, 1, 1]
    assert sc.geometric_fanout(4, 0, 0.7).tolist() == [0, 0, 0, 0, 0]
    for g, tot, a in ((8, 64, 0.6), (4, 33, 0.9), (1, 5, 0.2)):
        f = sc.geometric_fanout(g, tot, a)
        assert f.sum() == tot and np.all(np.diff(f) <= 0)
        exact = tot * a ** np.arange(g + 1) / np.sum(a ** np.arange(g + 1))
        assert np.all(np.abs(f - exact) < 1)


def test_closed_form_residual_order_and_support():
    # p proportional to id+1, q uniform: r_v = max((v+1)/S - 1/V, 0), S = V(V+1)/2,
    # decreasing in v, positive exactly for v + 1 > (V + 1) / 2
    V, g = 10, 1
    zt = np.stack([np.log(np.arange(1, V + 1, dtype=np.float64)), np.zeros(V)])[None]
    zd = np.zeros((1, 1, g, V))
    cand, w = sc.residual_topf(zt, zd, np.array([1.0], np.float32), [8, 0])
    assert cand[0, 0].tolist() == [9, 8, 7, 6, 5, -1, -1, -1]
    S = V * (V + 1) / 2
    np.testing.assert_allclose(w[0, 0, :5], [(v + 1) / S - 1 / V for v in (9, 8, 7, 6, 5)],
                               rtol=1e-13)


def test_brute_force_sort_of_normalised_weights():
    rng = np.random.default_rng(17)
    B, K, g, V = 3, 2, 3, 41
    zt = rng.normal(0, 1.5, size=(B, g + 1, V))
    zd = zt[:, None, :g] + rng.normal(0, 1.0, size=(B, K, g, V))
    zt[0, 1, 3] = zt[0, 1, 7] = zt[0, 1].max() + 1          # an exact tie in p
    T = np.array([0.6, 1.0, 1.4], np.float32)
    fan = [5, 4, 0, 3]
    cand, _ = sc.residual_topf(zt, zd, T, fan)
    for b in range(B):
        Tb = float(T[b])
        p = softmax(zt[b] / Tb, axis=-1)
        for k in range(K):
            off = 0
            for j, F in enumerate(fan):
                w = (np.maximum(p[j] - softmax(zd[b, k, j] / Tb), 0.0) if j < g else p[g])
                ranked = sorted((v for v in range(V) if w[v] > 0), key=lambda v: (-w[v], v))[:F]
                want = ranked + [-1] * (F - len(ranked))
                assert cand[b, k, off:off + F].tolist() == want, (b, k, j)
                off += F


def test_greedy_rows_rank_raw_target_logits():
    zt = np.array([[[1.0, 3.0, 3.0, 2.0], [0.0, 0.0, 5.0, -np.inf], [4.0, 1.0, 4.0, 4.0]]])
    zd = np.zeros((1, 1, 2, 4))
    cand, _ = sc.residual_topf(zt, zd, np.array([0.0], np.float32), [3, 4, 2])
    assert cand[0, 0].tolist() == [1, 2, 3, 2, 0, 1, -1, 0, 2]


def test_lookup_hand_cases():
    fan = [2, 1, 3]
    cand = np.array([[[5, 9, 7, 1, 2, 3]]])
    slots = sc.cache_lookup(cand, fan, np.array([[0]]), np.array([[9]]))
    assert slots.tolist() == [[1]]
    assert sc.cache_lookup(cand, fan, np.array([[1]]), np.array([[9]])).tolist() == [[-1]]
    assert sc.cache_lookup(cand, fan, np.array([[2]]), np.array([[3]])).tolist() == [[5]]
    assert sc.cache_lookup(cand, fan, np.array([[-1]]), np.array([[5]])).tolist() == [[-1]]
    assert sc.cache_lookup(cand, fan, np.array([[3]]), np.array([[5]])).tolist() == [[-1]]


# --- the pin to the method -------------------------------------------------------

G, V, N = 2, 12, 300_000
T32 = float(np.float32(0.9))
SEED = 0x5EED_CAC4E


def _rows():
    rng = np.random.default_rng(606)
    zt = rng.normal(0, 1.3, size=(G + 1, V))
    zd = zt[:G] + rng.normal(0, 1.0, size=(G, V))
    return zt, zd


def _predicted_hit_rate(zt, zd, fan, cand):
    p = softmax(zt / T32, axis=1)
    q = softmax(zd / T32, axis=1)
    alpha = oracle.acceptance_probability(zt[None], zd[None, None], np.array([T32], np.float32))
    law = oracle.outcome_law(alpha)[0, 0]
    rate, off = 0.0, 0
    for j, F in enumerate(fan):
        r = np.maximum(p[j] - q[j], 0.0) if j < G else p[G]
        ids = cand[off:off + F]
        rate += law[j] * r[ids[ids >= 0]].sum() / r.sum()
        off += F
    return rate


@pytest.fixture(scope="module")
def replicates():
    zt, zd = _rows()
    q = softmax(zd / T32, axis=1)
    rng = np.random.default_rng(31)
    toks = np.stack([rng.choice(V, size=N, p=q[j]) for j in range(G)], axis=1)
    out = oracle.verify(np.broadcast_to(zt, (N, G + 1, V)), np.broadcast_to(zd, (N, 1, G, V)),
                        toks[:, None, :], np.full(N, T32, dtype=np.float32), SEED,
                        np.zeros(N, dtype=np.int64))
    return out["accept_len"][:, 0], out["out_token"][:, 0]


def test_hit_rate_matches_the_law(replicates):
    zt, zd = _rows()
    fan = [4, 3, 2]
    cand, _ = sc.residual_topf(zt[None], zd[None, None], np.array([T32], np.float32), fan)
    n, y = replicates
    slots = sc.cache_lookup(np.broadcast_to(cand[0, 0], (N, 1, cand.shape[-1])), fan,
                            n[:, None], y[:, None])[:, 0]
    hit = np.mean(slots >= 0)
    want = _predicted_hit_rate(zt, zd, fan, cand[0, 0])
    assert 0.2 < want < 0.95
    assert abs(hit - want) < 5 * np.sqrt(want * (1 - want) / N), (hit, want)
    # the first candidate of every outcome is its most frequent emitted token
    off = 0
    for j, F in enumerate(fan):
        sel = n == j
        assert np.bincount(y[sel], minlength=V).argmax() == cand[0, 0, off]
        off += F


def test_planted_mistake_fails(replicates):
    # candidates ranked by p instead of the residual max(p - q, 0)
    zt, zd = _rows()
    fan = [4, 3, 2]
    wrong = []
    p = softmax(zt / T32, axis=1)
    for j, F in enumerate(fan):
        wrong += sorted(range(V), key=lambda v: (-p[j][v], v))[:F]
    wrong = np.array(wrong)
    n, y = replicates
    slots = sc.cache_lookup(np.broadcast_to(wrong, (N, 1, wrong.size)), fan, n[:, None],
                            y[:, None])[:, 0]
    cand, _ = sc.residual_topf(zt[None], zd[None, None], np.array([T32], np.float32), fan)
    want = _predicted_hit_rate(zt, zd, fan, cand[0, 0])
    assert abs(np.mean(slots >= 0) - want) > 10 * np.sqrt(want * (1 - want) / N)
