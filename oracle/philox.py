"""Philox4x32-10 counter-based generator, uniform and Gumbel maps (oracle side).

TEST INFRASTRUCTURE (see the package docstring): nothing on the product path
imports this module.

Philox4x32-10 is the generator of Salmon, Moraes, Dror and Shaw, "Parallel
Random Numbers: As Easy as 1, 2, 3" (SC'11). A block maps a 128-bit counter
(four 32-bit words) and a 64-bit key (two words) through ten rounds. Each
round multiplies words 0 and 2 by two fixed 32-bit multipliers, keeps the high
and low halves of the 64-bit products, and mixes the high halves with the
other two words and the round key; the key is advanced by two Weyl constants
between rounds.

Counter layout used by the verification (the pages only say that the accept
uniforms and the sampling noise come from a stream keyed by seed, batch row and
position):
    key     = (seed mod 2^32, seed >> 32)
    counter = (c0, position mod 2^32, chain row r = b*K + k, purpose)
    accept uniform of draft position j : c0 = 0,       word 0,     purpose ACCEPT
    sampling noise for vocabulary id v  : c0 = v >> 2,  word v & 3, purpose SAMPLE
"""

from __future__ import annotations

import numpy as np

MULT0 = 0xD2511F53
MULT1 = 0xCD9E8D57
WEYL0 = 0x9E3779B9
WEYL1 = 0xBB67AE85
ROUNDS = 10
_MASK = np.uint64(0xFFFFFFFF)
_SHIFT = np.uint64(32)


def block(c0, c1, c2, c3, k0, k1):
    """Philox4x32-10 of counter (c0, c1, c2, c3) under key (k0, k1).

    Arguments broadcast against each other; returns four uint32 arrays.
    Arithmetic is done in uint64, where a product of two 32-bit values is exact.
    """
    x0, x1, x2, x3, ka, kb = (np.asarray(a, dtype=np.uint64) & _MASK
                              for a in (c0, c1, c2, c3, k0, k1))
    x0, x1, x2, x3, ka, kb = np.broadcast_arrays(x0, x1, x2, x3, ka, kb)
    m0 = np.uint64(MULT0)
    m1 = np.uint64(MULT1)
    for rnd in range(ROUNDS):
        if rnd:
            ka = (ka + np.uint64(WEYL0)) & _MASK
            kb = (kb + np.uint64(WEYL1)) & _MASK
        p0 = m0 * x0
        p1 = m1 * x2
        hi0, lo0 = p0 >> _SHIFT, p0 & _MASK
        hi1, lo1 = p1 >> _SHIFT, p1 & _MASK
        x0, x1, x2, x3 = hi1 ^ x1 ^ ka, lo1, hi0 ^ x3 ^ kb, lo0
    return tuple(a.astype(np.uint32) for a in (x0, x1, x2, x3))


def key_of(seed: int):
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & 0xFFFFFFFF, seed >> 32


def uniform(word) -> np.ndarray:
    """Top 23 bits of a 32-bit word, centred: u = (floor(w / 2^9) + 1/2) * 2^-23.

    Every value lies strictly inside (0, 1) and is exact in float32 and float64.
    """
    w = np.asarray(word, dtype=np.uint32)
    return ((w >> np.uint32(9)).astype(np.float64) + 0.5) * 2.0 ** -23


def neg_log_uniform(u) -> np.ndarray:
    """-ln u, evaluated as -log1p(u - 1) for u >= 1/2 where u - 1 is exact."""
    u = np.asarray(u, dtype=np.float64)
    return np.where(u >= 0.5, -np.log1p(u - 1.0), -np.log(u))


def gumbel(u) -> np.ndarray:
    """Standard Gumbel noise G = -ln(-ln u)."""
    return -np.log(neg_log_uniform(u))


def accept_words(seed: int, chain_row, position, purpose: int):
    """Word 0 of the block keyed (seed; 0, position, chain_row, purpose)."""
    k0, k1 = key_of(seed)
    pos = np.asarray(position, dtype=np.int64) & 0xFFFFFFFF
    return block(0, pos, chain_row, purpose, k0, k1)[0]


def vocab_words(seed: int, chain_row, position, purpose: int, V: int):
    """One word per vocabulary id v in [0, V): word v & 3 of block (v >> 2, position, chain_row, purpose).

    chain_row and position are arrays of shape [C]; the result has shape [C, V].
    """
    k0, k1 = key_of(seed)
    r = np.asarray(chain_row, dtype=np.int64)[:, None]
    pos = (np.asarray(position, dtype=np.int64) & 0xFFFFFFFF)[:, None]
    nblk = (V + 3) // 4
    c0 = np.arange(nblk, dtype=np.int64)[None, :]
    w = np.stack(block(c0, pos, r, purpose, k0, k1), axis=-1)  # [C, nblk, 4]
    return w.reshape(w.shape[0], nblk * 4)[:, :V]
