"""Pins for the oracle's branch pruning (CPU only). Parity unpinned with respect
to the pages (they give no rule); the prefix sums and the ranking are pinned to
their definitions: hand cases, and a brute-force enumeration of every ordering."""
import itertools

import numpy as np

from oracle import branch_pruning as bp


def test_hand_case():
    logq = np.log(np.array([[[0.9, 0.8, 0.5],     # c = ln .9, ln .72, ln .36
                             [0.5, 0.9, 0.9],     # c = ln .5, ln .45, ln .405
                             [0.95, 0.95, 0.2],   # c = ln .95, ln .9025, ln .1805
                             [0.1, 0.9, 0.9]]]))  # c = ln .1 ...
    mask, L, c = bp.keep_branches(logq, np.log(0.4), 2)
    np.testing.assert_allclose(np.exp(c[0, 0]), [0.9, 0.72, 0.36])
    assert L[0].tolist() == [2, 3, 2, 0]
    # branch 1 (L = 3) first; branches 0 and 2 tie at L = 2: 0.9025 > 0.72 keeps branch 2
    assert mask[0].tolist() == [False, True, True, False]


def test_ranking_by_brute_force():
    rng = np.random.default_rng(4)
    for _ in range(50):
        K, g = 4, 3
        logq = np.log(rng.choice([0.2, 0.5, 0.9, 1.0], size=(1, K, g)))
        log_tau = np.log(rng.choice([0.1, 0.3, 0.6]))
        keep = int(rng.integers(1, K + 1))
        mask, L, c = bp.keep_branches(logq, log_tau, keep)
        # among all orderings, the kept set is the prefix of the lexicographically smallest key list
        best = None
        for perm in itertools.permutations(range(K)):
            keys = [(-L[0, k], -(c[0, k, L[0, k] - 1] if L[0, k] else -np.inf), k) for k in perm]
            if best is None or keys < best[0]:
                best = (keys, perm)
        assert set(np.nonzero(mask[0])[0]) == set(best[1][:keep])
        assert mask[0].sum() == keep


def test_prefix_is_leading_and_monotone():
    rng = np.random.default_rng(9)
    logq = -rng.exponential(0.5, size=(6, 3, 8))
    c = bp.branch_confidence(logq)
    assert np.all(np.diff(c, axis=-1) <= 0)
    L = bp.confident_prefix(c, np.log(0.2))
    for idx in np.ndindex(*L.shape):
        assert np.all(c[idx][:L[idx]] >= np.log(0.2)) and np.all(c[idx][L[idx]:] < np.log(0.2))
