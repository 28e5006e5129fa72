"""Batched speculative-sampling verification in float64 (oracle side).

TEST INFRASTRUCTURE (see the package docstring): nothing on the product path
imports this module.

What is computed, for every chain (b, k) -- batch row b, draft branch k, chain
row r = b*K + k -- from target logits z_t[b, 0..gamma, :] and draft logits
z_d[b, k, 0..gamma-1, :] with draft tokens x_0..x_{gamma-1}:

1. Temperature first: s = z / T_b, then ln Z = ln sum_v exp(s_v) per row
   (FlashSpec, technical summary, section 1 "On-device verification kernel",
   numerical-stability paragraph: temperature scaling goes before the
   log-softmax, and the arithmetic stays in log space).
2. Gather: ln p_j = s_t[j, x_j] - ln Z_t[j], ln q_j = s_d[j, x_j] - ln Z_d[j]
   (FlashSpec section 1, mechanism paragraph: two log-probability scalars per
   candidate, one from each model).
3. Accept test per position: accept_j iff ln u_j < ln p_j - ln q_j, i.e.
   u_j < min(1, p_j / q_j) since u_j < 1 (FlashSpec problem definition:
   per-token accept/reject). n = number of leading accepts.
4. n < gamma: correction token drawn from the residual max(p_n - q_n, 0)
   (Speculative Speculative Decoding, technical summary section 2,
   optimisation 2 "Saguaro sampling"; SpecTr-GBV section 2, termination
   step). n = gamma: bonus token drawn from p_gamma (SpecTr-GBV, same step).
   Both draws are Gumbel-max: argmax_v (ln w_v + G_v) with G_v standard
   Gumbel noise from the Philox stream, ties to the lowest id.
5. T_b = 0 (greedy): accept_j iff x_j is the target row's argmax (lowest id on
   ties); the emitted token is the argmax of target row n.

Readings where the pages are silent (each is listed in the design doc):
* the draft distribution uses the same per-row temperature as the target;
* an empty residual support (reachable only through rounding) falls back to a
  draw from p_n with the same noise;
* a needed row whose largest logit is not finite (every entry -inf, or any
  +inf or NaN entry) is an input error of its chains;
* decisions after the first rejection are computed but do not matter;
* greedy rows report ln Z_t = max_v z (the T -> 0 limit of T * ln Z),
  ln p in {0, -inf} and ln q = 0, so the scalar accept test reproduces them;
* a decision is "within eps of its threshold" when a perturbation of at most
  eps (1e-6) in any log-probability difference or perturbed score it depends
  on could change it; such chains are flagged.
"""

from __future__ import annotations

import numpy as np

from . import philox

ACCEPT = 0
SAMPLE = 1
FLAG_EPS = 1e-6

ERR_TOKEN = 1   # a draft token outside [0, V)
ERR_TEMP = 2    # temperature negative or NaN
ERR_ROW = 4     # a needed row whose largest logit is not finite: all -inf, +inf or NaN


def decode_logits(raw, dtype: str) -> np.ndarray:
    """Stored logits -> float64, exactly: bf16 bits widen to float32 by a 16-bit shift."""
    raw = np.asarray(raw)
    if dtype == "f32":
        return raw.astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.ascontiguousarray(raw).view(np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def scaled_logits(z: np.ndarray, T) -> np.ndarray:
    """Logits divided by the temperature, before any normalisation."""
    return z / T


def log_normalizer(s: np.ndarray) -> np.ndarray:
    """ln sum_v exp(s_v) over the last axis with the row maximum factored out.

    A row that is entirely -inf gives -inf. A row holding a NaN or a +inf has no
    normaliser (ln p of its +inf entry would be inf - inf): NaN.
    """
    m = np.max(s, axis=-1)
    finite = np.isfinite(m)
    m0 = np.where(finite, m, 0.0)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        total = np.sum(np.exp(s - m0[..., None]), axis=-1)
        out = m0 + np.log(total)
    return np.where(finite, out, np.where(np.isneginf(m), m, np.nan))


def normalize_rows(z: np.ndarray, T) -> tuple[np.ndarray, np.ndarray]:
    """Per row: ln Z = ln sum exp(z / T) for T > 0, max z for T = 0, NaN otherwise;
    and the argmax of the raw logits (lowest id on ties)."""
    T = np.asarray(T, dtype=np.float64)
    sampled = T > 0
    greedy = T == 0
    Tsafe = np.where(sampled, T, 1.0)
    lnz_sampled = log_normalizer(scaled_logits(z, Tsafe[..., None]))
    zmax = np.max(z, axis=-1)
    lnz = np.where(sampled, lnz_sampled, np.where(greedy, zmax, np.nan))
    return lnz, np.argmax(z, axis=-1)


def accept_uniforms(seed: int, chain_rows: np.ndarray, positions: np.ndarray) -> np.ndarray:
    """u for each (chain row, position): word 0 of Philox block (0, position, r, ACCEPT)."""
    return philox.uniform(philox.accept_words(seed, chain_rows, positions, ACCEPT))


def log_uniform(u) -> np.ndarray:
    return -philox.neg_log_uniform(u)


def accept_decisions(lp, lq, log_u) -> np.ndarray:
    """accept iff ln u < ln p - ln q; a NaN difference (both -inf) rejects."""
    with np.errstate(invalid="ignore"):
        return log_u < (lp - lq)


def first_rejection(accepted: np.ndarray) -> np.ndarray:
    """Number of leading accepts along the last axis (gamma when all accept)."""
    g = accepted.shape[-1]
    return np.where(accepted.all(axis=-1), g, np.argmin(accepted, axis=-1))


def residual_log_weights(lp: np.ndarray, lq: np.ndarray) -> np.ndarray:
    """ln max(p - q, 0) = ln p + ln(1 - q/p) where p > q, -inf elsewhere."""
    d = lq - lp
    with np.errstate(invalid="ignore", divide="ignore"):
        return np.where(d < 0, lp + np.log(-np.expm1(np.minimum(d, 0.0))), -np.inf)


def _residual_factor(d: np.ndarray) -> np.ndarray:
    with np.errstate(invalid="ignore", divide="ignore"):
        return np.where(d < 0, np.log(-np.expm1(np.minimum(d, 0.0))), -np.inf)


def sampling_noise(seed: int, chain_rows, positions, V: int) -> np.ndarray:
    """Gumbel noise G[c, v] from word v & 3 of Philox block (v >> 2, position_c, r_c, SAMPLE)."""
    return philox.gumbel(philox.uniform(philox.vocab_words(seed, chain_rows, positions, SAMPLE, V)))


def gumbel_argmax(scores: np.ndarray) -> np.ndarray:
    return np.argmax(scores, axis=-1)


def target_row_for(n: np.ndarray) -> np.ndarray:
    """Target row j verifies draft token j; after n accepts, row n supplies the next token."""
    return n


def bonus_row_for(g: int) -> int:
    """When all gamma drafts are accepted, the extra target row gamma supplies the bonus token."""
    return g


def bonus_scores(zt_last: np.ndarray, T: np.ndarray) -> np.ndarray:
    """Unnormalised log-weights of the bonus draw: ln p_gamma up to a constant."""
    return scaled_logits(zt_last, T[:, None])


def accept_from_logprobs(lp, lq, seed: int, pos0, batch_index=None):
    """The scalar-only path: decisions from given ln p, ln q of shape [B, K, gamma].

    Returns (accept_len [B, K], accept_bits [B, K] uint32, margin [B, K, gamma]).
    """
    lp = np.asarray(lp, dtype=np.float64)
    lq = np.asarray(lq, dtype=np.float64)
    B, K, g = lp.shape
    b = np.arange(B) if batch_index is None else np.asarray(batch_index)
    r = (b[:, None] * K + np.arange(K)[None, :])[:, :, None]
    pos = (np.asarray(pos0, dtype=np.int64)[:, None] + np.arange(g)[None, :])[:, None, :]
    log_u = log_uniform(accept_uniforms(seed, r, pos))
    acc = accept_decisions(lp, lq, log_u)
    bits = np.sum(acc.astype(np.uint64) << np.arange(g, dtype=np.uint64), axis=-1).astype(np.uint32)
    with np.errstate(invalid="ignore"):
        margin = (lp - lq) - log_u
    return first_rejection(acc), bits, margin


def sample_tokens(target, draft, T, lnz_t, lnz_d, argmax_t, n, seed: int, pos0, chain_rows,
                  eps: float = FLAG_EPS):
    """Emitted token of every chain given its accept length n.

    target [B, g+1, V], draft [B, K, g, V] (float64), T [B], lnz_t [B, g+1],
    lnz_d [B, K, g], argmax_t [B, g+1], n [B, K], chain_rows [B, K].
    Returns (token [B, K] int64, flagged [B, K] bool, empty_support [B, K] bool).
    """
    B, G1, V = target.shape
    g = G1 - 1
    K = draft.shape[1]
    T = np.asarray(T, dtype=np.float64)
    n = np.asarray(n, dtype=np.int64)
    token = np.full((B, K), -1, dtype=np.int64)
    flagged = np.zeros((B, K), dtype=bool)
    empty = np.zeros((B, K), dtype=bool)
    bb, kk = np.meshgrid(np.arange(B), np.arange(K), indexing="ij")
    pos0 = np.asarray(pos0, dtype=np.int64)

    greedy = (T[bb] == 0) & (n >= 0) & (n <= g)
    token[greedy] = argmax_t[bb[greedy], n[greedy]]

    res = (T[bb] > 0) & (n >= 0) & (n < g)
    if res.any():
        b, k, nn = bb[res], kk[res], n[res]
        Tc = T[b][:, None]
        # a row whose maximum is not finite gives NaN here; such rows are
        # input errors (verify sets their chains' outputs to -1)
        with np.errstate(invalid="ignore"):
            lp = scaled_logits(target[b, target_row_for(nn)], Tc) - lnz_t[b, target_row_for(nn)][:, None]
            lq = scaled_logits(draft[b, k, nn], Tc) - lnz_d[b, k, nn][:, None]
        logr = residual_log_weights(lp, lq)
        G = sampling_noise(seed, chain_rows[res], pos0[b] + nn, V)
        no_support = np.all(np.isneginf(logr), axis=-1)
        scores = np.where(no_support[:, None], lp + G, logr + G)
        y = gumbel_argmax(scores)
        rows = np.arange(len(y))
        # Robustness of the draw: each difference lq - lp and each score may be off by eps.
        with np.errstate(invalid="ignore"):
            d = lq - lp
            hi = lp + _residual_factor(d - eps) + G + eps
            lo_y = lp[rows, y] + _residual_factor(d[rows, y] + eps) + G[rows, y] - eps
            hi[rows, y] = -np.inf
            fl = np.max(hi, axis=-1) >= lo_y
            # Empty support (the draw from p_n): the emptiness itself is fragile when some
            # id sits within eps of the support (lq - lp < eps), and the draw from p_n is
            # fragile when its runner-up is within 2 eps, as for the bonus draw.
            near = np.any(d < eps, axis=-1)
            ps = lp + G
            best = ps[rows, y]
            ps[rows, y] = -np.inf
            fl_empty = near | (np.max(ps, axis=-1) >= best - 2 * eps)
        token[res] = y
        flagged[res] = np.where(no_support, fl_empty, fl)
        empty[res] = no_support

    bon = (T[bb] > 0) & (n == g)
    if bon.any():
        b = bb[bon]
        scores = (bonus_scores(target[b, bonus_row_for(g)], T[b])
                  + sampling_noise(seed, chain_rows[bon], pos0[b] + g, V))
        y = gumbel_argmax(scores)
        rows = np.arange(len(y))
        best = scores[rows, y]
        scores[rows, y] = -np.inf
        token[bon] = y
        flagged[bon] = np.max(scores, axis=-1) >= best - 2 * eps
    return token, flagged, empty


def verify(target, draft, tokens, temperature, seed: int, pos0, batch_index=None,
           dtype: str | None = None, eps: float = FLAG_EPS) -> dict:
    """Full verification step for a batch of rows.

    target [B, gamma+1, V], draft [B, K, gamma, V]: float64 logits, or stored
    logits when `dtype` ("f32"/"bf16") is given. tokens [B, K, gamma],
    temperature [B], pos0 [B]. batch_index [B] gives the global batch row of
    each row (default 0..B-1), so a subset of a large batch can be checked.
    """
    if dtype is not None:
        target = decode_logits(target, dtype)
        draft = decode_logits(draft, dtype)
    target = np.asarray(target, dtype=np.float64)
    draft = np.asarray(draft, dtype=np.float64)
    tokens = np.asarray(tokens, dtype=np.int64)
    B, G1, V = target.shape
    g = G1 - 1
    K = draft.shape[1]
    T = np.asarray(temperature, dtype=np.float32).astype(np.float64)
    pos0 = np.asarray(pos0, dtype=np.int64)
    bidx = np.arange(B) if batch_index is None else np.asarray(batch_index, dtype=np.int64)
    chain_rows = bidx[:, None] * K + np.arange(K)[None, :]

    sampled = T > 0
    greedy = T == 0
    lnz_t, argmax_t = normalize_rows(target, T[:, None])
    Td = np.where(sampled, T, np.nan)[:, None, None]
    lnz_d, _ = normalize_rows(draft, Td)

    tok_ok = (tokens >= 0) & (tokens < V)
    tok = np.where(tok_ok, tokens, 0)
    bb = np.arange(B)[:, None, None]
    kk = np.arange(K)[None, :, None]
    jj = np.arange(g)[None, None, :]
    Ts = np.where(sampled, T, 1.0)[:, None, None]
    with np.errstate(invalid="ignore"):
        lp_s = scaled_logits(target[bb, jj, tok], Ts) - lnz_t[bb, jj]
        lq_s = scaled_logits(draft[bb, kk, jj, tok], Ts) - lnz_d
    is_max = tok == argmax_t[bb, jj]
    gmask = greedy[:, None, None]
    lp = np.where(gmask, np.where(is_max, 0.0, -np.inf), lp_s)
    lq = np.where(gmask, 0.0, lq_s)

    pos = pos0[:, None, None] + jj
    log_u = log_uniform(accept_uniforms(seed, chain_rows[:, :, None], pos))
    acc = np.where(gmask, is_max, accept_decisions(lp, lq, log_u))
    n = first_rejection(acc)
    bits = np.sum(acc.astype(np.uint64) << np.arange(g, dtype=np.uint64), axis=-1).astype(np.uint32)
    with np.errstate(invalid="ignore"):
        margin = np.where(gmask, np.nan, (lp - lq) - log_u)

    token, sflag, empty = sample_tokens(target, draft, T, lnz_t, lnz_d, argmax_t, n, seed, pos0,
                                        chain_rows, eps)

    # Accept decisions that fixed n: positions 0..min(n, gamma-1).
    decided = jj <= np.minimum(n, g - 1)[:, :, None]
    with np.errstate(invalid="ignore"):
        aflag = np.any(decided & (np.abs(margin) < eps) & ~gmask, axis=-1)
    flagged = (aflag | sflag) & sampled[:, None]

    # Input errors: the chain's outputs become -1 and the error word gets a bit.
    err_chain = np.zeros((B, K), dtype=np.int64)
    err_chain |= np.where(~tok_ok.all(axis=-1), ERR_TOKEN, 0)
    err_chain |= np.where(~(sampled | greedy), ERR_TEMP, 0)[:, None]
    tmax = np.max(target, axis=-1)
    bad_t = np.any(~np.isfinite(tmax), axis=-1)         # -inf, +inf or NaN maximum
    dmax = np.max(draft, axis=-1)
    bad_d = np.any(~np.isfinite(dmax), axis=-1) & sampled[:, None]
    err_chain |= np.where(bad_t[:, None] | bad_d, ERR_ROW, 0)
    bad = err_chain != 0
    accept_len = np.where(bad, -1, n)
    token = np.where(bad, -1, token)

    lnz_d_out = np.where(sampled[:, None, None], lnz_d, np.nan)
    return dict(accept_len=accept_len, out_token=token, logp=lp, logq=lq,
                lnZ_target=lnz_t, lnZ_draft=lnz_d_out, argmax_target=argmax_t,
                accept_bits=bits, margin=margin, flagged=flagged & ~bad,
                empty_support=empty, error=int(np.bitwise_or.reduce(err_chain.ravel())),
                chain_error=err_chain)
