"""Confidence-based pruning of draft branches before verification (oracle side).

TEST INFRASTRUCTURE (see the package docstring): nothing on the product path
imports this module.

FlexDraft (technical summary, methodology component 3 "Flex decoding",
selective verification for small batches): with several draft branches per
row, the cumulative draft confidence of each branch estimates how far it will
be accepted; low-confidence branches are dropped and only a subset of
high-confidence prefixes is verified, without changing the draft length.

PARITY UNPINNED with respect to the pages: they give no rule. The reading
taken here (listed in the design doc):
* cumulative confidence c_k(j) = sum_{i <= j} ln q_k,i, the log of the draft's
  probability of branch k's first j + 1 tokens (ln q at the drafted tokens);
* the confident prefix of branch k is L_k = the number of positions with
  c_k(j) >= ln tau (c is non-increasing, so these are leading positions);
* a batch row keeps its `keep` branches of largest L_k, ties to the larger
  c_k(L_k - 1) (the whole-prefix confidence; -inf when L_k = 0), then to the
  lower k.
The prefix sum and the ranking are pinned to their definitions (hand cases and
a brute-force sort); the rule itself is not pinned to the pages.
"""

from __future__ import annotations

import numpy as np


def branch_confidence(logq) -> np.ndarray:
    """c [B, K, gamma]: running sums of ln q along the draft positions, in float64."""
    return np.cumsum(np.asarray(logq, dtype=np.float64), axis=-1)


def confident_prefix(conf, log_tau: float) -> np.ndarray:
    """L [B, K]: number of positions whose cumulative confidence is >= ln tau."""
    return np.sum(np.asarray(conf) >= log_tau, axis=-1)


def keep_branches(logq, log_tau: float, keep: int):
    """(keep_mask [B, K] bool, L [B, K], c [B, K, gamma]) under the rule above."""
    c = branch_confidence(logq)
    L = confident_prefix(c, log_tau)
    B, K, g = c.shape
    mask = np.zeros((B, K), dtype=bool)
    for b in range(B):
        def key(k):
            last = c[b, k, L[b, k] - 1] if L[b, k] > 0 else -np.inf
            return (-L[b, k], -last, k)
        for k in sorted(range(K), key=key)[:keep]:
            mask[b, k] = True
    return mask, L, c
