"""Residual top-F candidates per verification outcome, and the speculation-cache lookup.

TEST INFRASTRUCTURE (see the package docstring): nothing on the product path
imports this module.

Speculative Speculative Decoding (technical summary, "core mechanism", items 2
and 3; optimisation 1 "geometric fan-out"; optimisation 2 on the residual) keys a
cache by the verification outcome: how many drafts are accepted (n) and which
token the verifier emits after them (y, drawn from the residual
r_n = max(p_n - q_n, 0) when n < gamma, or from p_gamma when n = gamma). With a
budget of F_j candidate tokens for the outcome n = j, the cache holding the F_j
most likely y for every j is hit exactly when the emitted token is among those
of its n. The fan-out gives short accept lengths more candidates because long
ones are geometrically rarer.

Readings where the pages are silent (each is listed in the design doc):
* candidates of outcome j < gamma: the F_j ids of largest r_j, ties to the lowest
  id, ids with r_j = 0 excluded (the residual support may hold fewer than F_j);
  outcome gamma: the F_gamma ids of largest p_gamma;
* greedy rows (T = 0): the emitted token is the target row's argmax, so the
  candidates are the F_j largest raw target logits of row j (ties lowest id);
* geometric fan-out: F_j proportional to a^j (a in (0, 1]), rounded to integers
  summing to the budget by largest remainders (ties to the smaller j);
* a chain hits when its accept length n is valid and its emitted token is among
  the candidates of outcome n; the lookup reports the slot, or -1.
"""

from __future__ import annotations

import numpy as np

from .acceptance import row_probabilities
from .specverify import decode_logits


def geometric_fanout(gamma: int, total: int, ratio: float) -> np.ndarray:
    """F_0..F_gamma summing to `total`, proportional to ratio**j (largest remainders)."""
    share = ratio ** np.arange(gamma + 1, dtype=np.float64)
    exact = total * share / share.sum()
    base = np.floor(exact).astype(np.int64)
    left = int(total - base.sum())
    order = sorted(range(gamma + 1), key=lambda j: (-(exact[j] - base[j]), j))
    for j in order[:left]:
        base[j] += 1
    return base


def outcome_weights(target, draft, temperature, dtype: str | None = None) -> np.ndarray:
    """[B, K, gamma+1, V] ranking weights of the emitted token for each outcome n = j:
    r_j = max(p_j - q_j, 0) (j < gamma), p_gamma (j = gamma); greedy rows: raw target
    logits (-inf = excluded)."""
    if dtype is not None:
        target = decode_logits(target, dtype)
        draft = decode_logits(draft, dtype)
    zt = np.asarray(target, dtype=np.float64)
    zd = np.asarray(draft, dtype=np.float64)
    B, K, g, V = zd.shape
    T = np.asarray(temperature, dtype=np.float32).astype(np.float64)
    sampled = T > 0
    Ts = np.where(sampled, T, 1.0)
    p = row_probabilities(zt, Ts[:, None])                    # [B, g+1, V]
    q = row_probabilities(zd, Ts[:, None, None])              # [B, K, g, V]
    w = np.empty((B, K, g + 1, V))
    w[:, :, :g] = np.maximum(p[:, None, :g] - q, 0.0)
    w[:, :, g] = p[:, None, g]
    # outcomes of weight 0 are not candidates
    w = np.where(w > 0, w, -np.inf)
    greedy_w = np.broadcast_to(zt[:, None], (B, K, g + 1, V))
    return np.where(sampled[:, None, None, None], w, greedy_w)


def residual_topf(target, draft, temperature, fanout, dtype: str | None = None):
    """cand [B, K, sum F] int64 (-1 padding) and their weights, outcome-major.

    Outcome j contributes F_j ids sorted by weight, largest first, ties to the
    lowest id; ids of weight -inf (excluded) are never listed."""
    w = outcome_weights(target, draft, temperature, dtype)
    B, K, G1, V = w.shape
    fanout = np.asarray(fanout, dtype=np.int64)
    total = int(fanout.sum())
    cand = np.full((B, K, total), -1, dtype=np.int64)
    cw = np.full((B, K, total), -np.inf)
    ids = np.arange(V)
    off = 0
    for j in range(G1):
        F = int(fanout[j])
        if F:
            wj = w[:, :, j]                                     # [B, K, V]
            order = np.lexsort((np.broadcast_to(ids, wj.shape), -wj), axis=-1)[..., :F]
            top_w = np.take_along_axis(wj, order, axis=-1)
            ok = top_w > -np.inf
            width = order.shape[-1]
            cand[:, :, off:off + width] = np.where(ok, order, -1)
            cw[:, :, off:off + width] = np.where(ok, top_w, -np.inf)
        off += F
    return cand, cw


def cache_lookup(cand, fanout, accept_len, out_token) -> np.ndarray:
    """Slot of each chain's emitted token among the candidates of its outcome, or -1."""
    cand = np.asarray(cand)
    fanout = np.asarray(fanout, dtype=np.int64)
    offs = np.concatenate([[0], np.cumsum(fanout)])
    n = np.asarray(accept_len)
    y = np.asarray(out_token)
    slot = np.full(n.shape, -1, dtype=np.int64)
    G1 = fanout.size
    for idx in np.ndindex(*n.shape):
        nn = int(n[idx])
        if 0 <= nn < G1 and y[idx] >= 0:
            seg = cand[idx][offs[nn]:offs[nn + 1]]
            hit = np.nonzero(seg == y[idx])[0]
            if hit.size:
                slot[idx] = offs[nn] + int(hit[0])
    return slot
