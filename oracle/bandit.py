"""Online bandit draft selection: UCB1 and Thompson sampling (oracle side).

TEST INFRASTRUCTURE (see the package docstring): nothing on the product path
imports this module.

FlashSpec (technical summary, section 2 "Online bandit draft selection") treats
the choice among K draft models as a K-armed bandit: each decoding step picks
one arm from its past performance, the reward is the accepted fraction of the
step's draft tokens, and the policies are UCB1 and Thompson sampling; the
policy depends only on past acceptance history, so the output distribution is
unchanged.

* UCB1 (Auer, Cesa-Bianchi and Fischer, "Finite-time analysis of the
  multiarmed bandit problem", 2002): play every arm once (lowest index
  first), then the arm maximising mean_i + sqrt(c ln t / n_i), t = pulls so
  far, n_i = pulls of arm i, c = 2 in the paper; ties to the lowest index.
* Thompson sampling (Thompson 1933; Agrawal and Goyal 2012 for Bernoulli
  rewards): draw theta_i ~ Beta(1 + S_i, 1 + n_i - S_i), S_i = sum of arm i's
  rewards, and play the largest (ties to the lowest index).

Readings where the pages are silent (listed in the design doc): the reward of a step
is sum(accept_len) / (chains * gamma); a fractional reward enters the Beta
posterior as fractional pseudo-counts; Beta draws are X / (X + Y) with X, Y
Gamma variates by Marsaglia and Tsang's method ("A simple method for
generating gamma variables", 2000; shapes here are >= 1), whose normals come
from the Box-Muller transform; every uniform is a double built from two
32-bit words of Philox4x32-10 keyed by the seed, with counter
(t, arm, (g << 16) | attempt, 2) for draw t, arm, variate g in {0, 1}.
"""

from __future__ import annotations

import math

import numpy as np

from . import philox

UCB1 = 0
THOMPSON = 1
PURPOSE_BANDIT = 2
MAX_ATTEMPTS = 1000


def step_reward(accept_len, gamma: int) -> float:
    """Accepted fraction of a step's draft tokens: sum(n) / (chains * gamma)."""
    n = np.asarray(accept_len)
    return float(np.sum(np.clip(n, 0, gamma))) / (n.size * gamma)


def _uniform53(w0: int, w1: int) -> float:
    """(floor(w0 / 2^5) * 2^26 + floor(w1 / 2^6) + 1/2) * 2^-53: strictly inside (0, 1)."""
    return ((w0 >> 5) * 67108864.0 + (w1 >> 6) + 0.5) * (1.0 / 9007199254740992.0)


def _block(seed: int, t: int, arm: int, g: int, attempt: int):
    out = philox.block(np.uint32(t & 0xFFFFFFFF), np.uint32(arm), np.uint32((g << 16) | attempt),
                       np.uint32(PURPOSE_BANDIT), np.uint32(seed & 0xFFFFFFFF),
                       np.uint32((seed >> 32) & 0xFFFFFFFF))
    return [int(x) for x in out]


def gamma_variate(shape: float, seed: int, t: int, arm: int, g: int) -> float:
    """Gamma(shape, 1) for shape >= 1 by Marsaglia-Tsang, one Philox block per attempt."""
    d = shape - 1.0 / 3.0
    c = 1.0 / math.sqrt(9.0 * d)
    for attempt in range(MAX_ATTEMPTS):
        w = _block(seed, t, arm, g, attempt)
        u1 = _uniform53(w[0], w[1])
        u2 = _uniform53(w[2], w[3])
        # Box-Muller normal from (u1, u2), then the acceptance uniform from the next block
        x = math.sqrt(-2.0 * math.log(u1)) * math.cos(2.0 * math.pi * u2)
        v = 1.0 + c * x
        if v <= 0.0:
            continue
        v = v * v * v
        wa = _block(seed, t, arm, g, attempt + MAX_ATTEMPTS)
        u = _uniform53(wa[0], wa[1])
        x2 = x * x
        if u < 1.0 - 0.0331 * x2 * x2:
            return d * v
        if math.log(u) < 0.5 * x2 + d * (1.0 - v + math.log(v)):
            return d * v
    return d  # unreachable in practice (acceptance > 0.95 per attempt)


def beta_variate(a: float, b: float, seed: int, t: int, arm: int) -> float:
    x = gamma_variate(a, seed, t, arm, 0)
    y = gamma_variate(b, seed, t, arm, 1)
    return x / (x + y)


class Bandit:
    """The selector's state: pulls and reward sums per arm, and the step counter."""

    def __init__(self, arms: int, policy: int, seed: int = 0, c: float = 2.0):
        self.arms, self.policy, self.seed, self.c = arms, policy, seed, c
        self.pulls = [0] * arms
        self.sums = [0.0] * arms
        self.t = 0          # pulls so far
        self.draws = 0      # Thompson selections so far

    def select(self) -> int:
        if self.policy == UCB1:
            for i in range(self.arms):
                if self.pulls[i] == 0:
                    return i
            best, bi = -math.inf, 0
            for i in range(self.arms):
                idx = self.sums[i] / self.pulls[i] + math.sqrt(self.c * math.log(self.t) / self.pulls[i])
                if idx > best:
                    best, bi = idx, i
            return bi
        best, bi = -math.inf, 0
        for i in range(self.arms):
            theta = beta_variate(1.0 + self.sums[i], 1.0 + self.pulls[i] - self.sums[i], self.seed,
                                 self.draws, i)
            if theta > best:
                best, bi = theta, i
        self.draws += 1
        return bi

    def update(self, arm: int, reward: float) -> None:
        self.pulls[arm] += 1
        self.sums[arm] += reward
        self.t += 1
