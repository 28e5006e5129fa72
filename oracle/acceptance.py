"""Exact acceptance probability per draft position and the law of the accept length.

TEST INFRASTRUCTURE (see the package docstring): nothing on the product path
imports this module.

What is computed, for every chain (b, k) and draft position j < gamma, from the
target row z_t[b, j] and the draft row z_d[b, k, j] at the row's temperature T:

* alpha_j = sum_v min(p_j(v), q_j(v)), with p_j = softmax(z_t[b, j] / T) and
  q_j = softmax(z_d[b, k, j] / T). It is the probability that the accept test
  passes at position j when the draft token is drawn from q_j:
  sum_x q(x) min(1, p(x) / q(x)) = sum_x min(p(x), q(x)). (FlashSpec, technical
  summary, section 2 "Online bandit draft selection": the reward is the
  accepted fraction of draft tokens; Speculative Speculative Decoding,
  technical summary, optimisation 1 "geometric fan-out": verified lengths fall
  off geometrically. Both use this per-position acceptance rate.)
* With the positions' accept events independent, the accept length n is
      P(n = m) = alpha_0 ... alpha_{m-1} (1 - alpha_m)   for m < gamma,
      P(n = gamma) = alpha_0 ... alpha_{gamma-1}.
  (Speculative Speculative Decoding, same passage: the distribution behind the
  fan-out; SpecTr-GBV and FlashSpec: n is the number of leading accepts.)

Readings where the pages are silent (each is listed in the design doc):
* the draft distribution uses the target row's temperature (as in the step);
* greedy rows (T = 0): p_j and q_j are point masses at the rows' lowest-id
  argmaxes, so alpha_j is 1 when the two argmaxes coincide and 0 otherwise
  (the accept rule of a greedy row with a greedy draft);
* a negative or NaN temperature gives NaN.
"""

from __future__ import annotations

import numpy as np

from .specverify import decode_logits, log_normalizer, scaled_logits


def row_probabilities(z: np.ndarray, T: np.ndarray) -> np.ndarray:
    """softmax(z / T) over the last axis in float64; T broadcasts against z[..., 0]."""
    s = scaled_logits(z, T[..., None])
    lnz = log_normalizer(s)
    with np.errstate(invalid="ignore", over="ignore"):
        return np.exp(s - lnz[..., None])


def acceptance_probability(target, draft, temperature, dtype: str | None = None) -> np.ndarray:
    """alpha [B, K, gamma] from target [B, gamma+1, V] and draft [B, K, gamma, V]."""
    if dtype is not None:
        target = decode_logits(target, dtype)
        draft = decode_logits(draft, dtype)
    zt = np.asarray(target, dtype=np.float64)
    zd = np.asarray(draft, dtype=np.float64)
    B, K, g, V = zd.shape
    T = np.asarray(temperature, dtype=np.float32).astype(np.float64)
    sampled = T > 0
    greedy = T == 0
    Ts = np.where(sampled, T, 1.0)

    p = row_probabilities(zt[:, :g], Ts[:, None])             # [B, g, V]
    q = row_probabilities(zd, Ts[:, None, None])               # [B, K, g, V]
    alpha_s = np.sum(np.minimum(p[:, None], q), axis=-1)       # [B, K, g]

    same = np.argmax(zt[:, :g], axis=-1)[:, None, :] == np.argmax(zd, axis=-1)
    alpha_g = same.astype(np.float64)

    return np.where(sampled[:, None, None], alpha_s,
                    np.where(greedy[:, None, None], alpha_g, np.nan))


def outcome_law(alpha) -> np.ndarray:
    """P(n = m) for m = 0..gamma, shape [..., gamma + 1], from alpha [..., gamma]."""
    alpha = np.asarray(alpha, dtype=np.float64)
    g = alpha.shape[-1]
    reach = np.ones(alpha.shape[:-1] + (g + 1,), dtype=np.float64)   # P(n >= m)
    for m in range(1, g + 1):
        reach[..., m] = reach[..., m - 1] * alpha[..., m - 1]
    law = np.empty_like(reach)
    law[..., :g] = reach[..., :g] * (1.0 - alpha)
    law[..., g] = reach[..., g]
    return law


def expected_accept_length(law) -> np.ndarray:
    """E[n] = sum_m m P(n = m)."""
    law = np.asarray(law, dtype=np.float64)
    return np.sum(law * np.arange(law.shape[-1]), axis=-1)
