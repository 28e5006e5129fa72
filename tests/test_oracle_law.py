"""Pins for the oracle's accept test, residual and bonus draws (CPU only).

The law of the emitted tokens is fixed by mathematics: with context-free
target distributions p_0..p_gamma and draft distributions q_0..q_{gamma-1},
draft tokens x_j ~ q_j, the step emits x_0..x_{k-1} followed by y with
probability

    P(n = k, x_<k, y) = prod_{j<k} min(p_j, q_j)(x_j) * max(p_k - q_k, 0)(y)   (k < gamma)
    P(n = gamma, x, y) = prod_{j<gamma} min(p_j, q_j)(x_j) * p_gamma(y)

so each emitted token is distributed as the target alone would draw it (the
losslessness every page claims). The oracle is run on 10^6 replicates and its
outcome frequencies are compared with this law by a chi-square test at
alpha = 0.01 (FlashSpec, section 3 "Correctness and testing": a distribution-
equivalence gate at alpha = 0.01, and the lesson that large samples are needed
to see subtle shifts). Planted mistakes in the oracle -- temperature after the
log-softmax, residual replaced by p or q, off-by-one target row, bonus from the
wrong row -- must fail the same gate.
"""
import numpy as np
import pytest
from scipy import stats
from scipy.special import softmax

import oracle
import workloads
from oracle import philox
from oracle import specverify as sv

V, G = 8, 2
T32 = float(np.float32(0.7))
N_REPLICATES = 1_000_000
ALPHA = 0.01
SEED = 0x1234_5678_9ABC_DEF0


def _distributions():
    rng = np.random.default_rng(12345)
    zt = rng.normal(0, 1.5, size=(G + 1, V))
    zd = zt[:G] + rng.normal(0, 1.0, size=(G, V))
    return zt, zd, softmax(zt / T32, axis=1), softmax(zd / T32, axis=1)


def _exact_law(p, q):
    """Probability of every outcome (k, x_0..x_{k-1}, y), laid out k-major, base-V digits."""
    cells = []
    for k in range(G + 1):
        w = np.ones(1)
        for j in range(k):
            w = np.outer(w, np.minimum(p[j], q[j])).ravel()
        last = np.maximum(p[k] - q[k], 0.0) if k < G else p[G]
        cells.append(np.outer(w, last).ravel())
    return np.concatenate(cells)


def _cell_index(n, tokens, y):
    offsets = np.cumsum([0] + [V ** (k + 1) for k in range(G)])
    idx = np.zeros_like(n)
    for j in range(G):
        idx = np.where(j < n, idx * V + tokens[:, j], idx)
    idx = idx * V + y
    return offsets[n] + idx


def _run(N=N_REPLICATES, seed=SEED):
    zt, zd, p, q = _distributions()
    rng = np.random.default_rng(777)
    toks = np.stack([rng.choice(V, size=N, p=q[j]) for j in range(G)], axis=1)
    out = oracle.verify(np.broadcast_to(zt, (N, G + 1, V)), np.broadcast_to(zd, (N, 1, G, V)),
                        toks[:, None, :], np.full(N, T32, dtype=np.float32), seed,
                        np.zeros(N, dtype=np.int64))
    return out["accept_len"][:, 0], toks, out["out_token"][:, 0], p, q


def _chi2_pvalue(observed, expected_prob, N):
    exp = expected_prob * N
    small = exp < 5
    o = np.concatenate([observed[~small], [observed[small].sum()]])
    e = np.concatenate([exp[~small], [exp[small].sum()]])
    if e[-1] == 0:
        o, e = o[:-1], e[:-1]
    stat = np.sum((o - e) ** 2 / e)
    return stats.chi2.sf(stat, len(e) - 1)


@pytest.fixture(scope="module")
def replicates():
    return _run()


def test_exact_law_is_a_distribution():
    _, _, p, q = _distributions()
    law = _exact_law(p, q)
    assert np.isclose(law.sum(), 1.0, atol=1e-12)
    # P(accept at position j) = sum_v min(p_j, q_j)
    alpha0 = np.minimum(p[0], q[0]).sum()
    assert np.isclose(law[V:].sum(), alpha0, atol=1e-12)


def test_outcome_law_chi2_gate(replicates):
    n, toks, y, p, q = replicates
    law = _exact_law(p, q)
    counts = np.bincount(_cell_index(n, toks, y), minlength=law.size)
    assert counts.size == law.size
    pval = _chi2_pvalue(counts, law, N_REPLICATES)
    assert pval >= ALPHA, pval


def test_emitted_tokens_follow_the_target(replicates):
    n, toks, y, p, q = replicates
    first = np.where(n >= 1, toks[:, 0], y)
    assert _chi2_pvalue(np.bincount(first, minlength=V), p[0], N_REPLICATES) >= ALPHA
    sel = n >= 1
    second = np.where(n[sel] >= 2, toks[sel, 1], y[sel])
    assert _chi2_pvalue(np.bincount(second, minlength=V), p[1], int(sel.sum())) >= ALPHA
    sel = n == G
    assert _chi2_pvalue(np.bincount(y[sel], minlength=V), p[G], int(sel.sum())) >= ALPHA


def test_acceptance_rate_equals_overlap(replicates):
    n, _, _, p, q = replicates
    alpha0 = np.minimum(p[0], q[0]).sum()
    rate = np.mean(n >= 1)
    assert abs(rate - alpha0) < 5 * np.sqrt(alpha0 * (1 - alpha0) / N_REPLICATES)


def _t_after_log_softmax(orig):
    def wrong(z, T):
        T = np.asarray(T, dtype=np.float64)
        lnz1, am = orig(z, np.ones_like(T))
        return np.where(T > 0, lnz1 / np.where(T > 0, T, 1.0), lnz1), am
    return wrong


MUTATIONS = {
    "temperature_after_log_softmax": ("normalize_rows", _t_after_log_softmax),
    "residual_is_p": ("residual_log_weights", lambda orig: (lambda lp, lq: lp)),
    "residual_is_q": ("residual_log_weights", lambda orig: (lambda lp, lq: lq)),
    "off_by_one_target_row": ("target_row_for", lambda orig: (lambda n: n + 1)),
    "bonus_from_row_gamma_minus_1": ("bonus_row_for", lambda orig: (lambda g: g - 1)),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_fail_the_gate(name, monkeypatch):
    attr, make_wrong = MUTATIONS[name]
    monkeypatch.setattr(sv, attr, make_wrong(getattr(sv, attr)))
    n, toks, y, p, q = _run()
    law = _exact_law(p, q)
    pval = _chi2_pvalue(np.bincount(_cell_index(n, toks, y), minlength=law.size), law, N_REPLICATES)
    assert pval < ALPHA, f"mutation {name} passed the gate (p = {pval})"


def test_identical_distributions_accept_everything():
    w = workloads.make("c2", B=16)
    for d in (w.target[:, None, :-1].copy(),):
        for seed in (0, 1, 2 ** 63 + 5, 12345):
            out = oracle.verify(w.target, d, w.tokens, w.temperature, seed, w.pos0, dtype=w.dtype)
            assert np.all(out["accept_len"] == w.gamma)
            assert np.all(out["logp"] == out["logq"])


def test_draft_below_target_at_the_token_never_rejects():
    w = workloads.make("c3", B=6, V=4096)
    zt = sv.decode_logits(w.target, w.dtype)
    zd = np.repeat(zt[:, None, :-1], 1, axis=1).copy()
    bb, jj = np.meshgrid(np.arange(w.B), np.arange(w.gamma), indexing="ij")
    zd[bb, 0, jj, w.tokens[:, 0, :]] -= 0.75          # q(x_j) <= p(x_j) at every position
    for seed in range(5):
        out = oracle.verify(zt, zd, w.tokens, w.temperature, seed, w.pos0)
        assert np.all(out["accept_len"] == w.gamma)
        assert np.all(out["logp"] >= out["logq"])


def test_correction_differs_from_rejected_token():
    w = workloads.make("c3", B=32, V=2048)
    out = oracle.verify(w.target, w.draft, w.tokens, w.temperature, w.seed, w.pos0, dtype=w.dtype)
    n = out["accept_len"][:, 0]
    rej = n < w.gamma
    assert rej.any()
    assert np.all(out["out_token"][rej, 0] != w.tokens[rej, 0, n[rej]])


def test_residual_fixture(golden):
    fx = golden("residual_v3.json")
    p, q = np.array(fx["p"]), np.array(fx["q"])
    N = 20000
    for tok, pacc in fx["accept_probability"].items():
        tok = int(tok)
        out = oracle.verify(np.broadcast_to(np.log(np.stack([p, p])), (N, 2, 3)),
                            np.broadcast_to(np.log(q)[None, None, None, :], (N, 1, 1, 3)),
                            np.full((N, 1, 1), tok), np.full(N, fx["T"], dtype=np.float32),
                            99, np.arange(N))
        n = out["accept_len"][:, 0]
        rate = n.mean()
        assert abs(rate - pacc) <= 5 * np.sqrt(max(pacc * (1 - pacc), 1e-12) / N) + 1e-12
        assert np.all(out["out_token"][n == 0, 0] == fx["correction_token"])


def test_greedy_rows_ignore_seed_position_and_draft_logits(golden):
    w = workloads.make("c4", B=8, V=3000)
    base = oracle.verify(w.target, w.draft, w.tokens, w.temperature, w.seed, w.pos0, dtype=w.dtype)
    other = oracle.verify(w.target, w.draft[:, :, ::-1].copy(), w.tokens, w.temperature, 17,
                          w.pos0 + 1000, dtype=w.dtype)
    g = w.temperature == 0
    assert g.any()
    for key in ("accept_len", "out_token"):
        assert np.array_equal(base[key][g], other[key][g])
    zt = sv.decode_logits(w.target, w.dtype)
    am = np.argmax(zt, axis=-1)
    for b in np.flatnonzero(g):
        n = base["accept_len"][b, 0]
        assert np.array_equal(w.tokens[b, 0, :n], am[b, :n])
        assert n == w.gamma or w.tokens[b, 0, n] != am[b, n]
        assert base["out_token"][b, 0] == am[b, n]
    fx = golden("greedy_ties.json")
    z = np.array(fx["target_row"])
    for tok, want_n in ((fx["accepted_token"], 1), (fx["rejected_token"], 0)):
        out = oracle.verify(np.stack([z, z])[None], np.zeros((1, 1, 1, 4)), np.array([[[tok]]]),
                            np.zeros(1, np.float32), 0, np.zeros(1, int))
        assert out["accept_len"][0, 0] == want_n and out["out_token"][0, 0] == fx["argmax"]


def test_scalar_path_reproduces_the_full_path():
    for name, kw in (("c3", dict(B=16, V=4096)), ("c4", dict(B=16, V=4096)),
                     ("c5", dict(B=4, V=2048))):
        w = workloads.make(name, **kw)
        out = oracle.verify(w.target, w.draft, w.tokens, w.temperature, w.seed, w.pos0, dtype=w.dtype)
        n, bits, _ = oracle.accept_from_logprobs(out["logp"], out["logq"], w.seed, w.pos0)
        assert np.array_equal(n, out["accept_len"])
        assert np.array_equal(bits, out["accept_bits"])


def test_accept_flag_marks_decisions_within_eps():
    seed, pos = 31, 0
    u = sv.accept_uniforms(seed, np.array([0]), np.array([pos]))[0]
    if u <= 0.5:
        pytest.skip("pick a seed with u > 1/2")
    for off, flagged in ((5e-7, True), (-5e-7, True), (1e-5, False), (-1e-5, False)):
        # target [0, 0] (p = 1/2); draft [a, 0] with token 0: ln p - ln q = ln(1 + e^-a) - ln 2
        a = -np.log(2 * u * np.exp(off) - 1)
        out = oracle.verify(np.zeros((1, 2, 2)), np.array([[[[a, 0.0]]]]), np.array([[[0]]]),
                            np.ones(1, np.float32), seed, np.array([pos]))
        assert bool(out["flagged"][0, 0]) == flagged, off
        assert np.isclose(out["margin"][0, 0, 0], off, atol=1e-9)


def test_sampling_flag_marks_near_ties():
    seed, V2 = 8, 2
    G2 = sv.sampling_noise(seed, np.array([0]), np.array([1]), V2)[0]
    for off, flagged in ((1e-7, True), (1.5e-6, True), (3e-6, False), (-1e-5, False)):
        # gamma = 1, the draft token is accepted (p = q), then the bonus row draws between two
        # tokens whose perturbed scores differ by `off`
        s1 = 0.0 + G2[0] - G2[1] + off
        zt = np.array([[[0.0, 0.0], [0.0, s1]]])
        out = oracle.verify(zt, zt[:, None, :1], np.array([[[0]]]), np.ones(1, np.float32), seed,
                            np.array([0]))
        assert out["accept_len"][0, 0] == 1
        assert bool(out["flagged"][0, 0]) == flagged, off


def test_uniforms_are_keyed_by_seed_row_and_position():
    a = sv.accept_uniforms(3, np.arange(4)[:, None], np.arange(5)[None, :] + 10)
    assert len(np.unique(a)) == a.size
    b = sv.accept_uniforms(3, np.arange(4)[:, None], np.arange(5)[None, :] + 11)
    assert np.array_equal(a[:, 1:], b[:, :-1])     # position-keyed: shifting pos0 shifts the stream
    c = sv.accept_uniforms(4, np.arange(4)[:, None], np.arange(5)[None, :] + 10)
    assert not np.any(a == c)
    assert np.array_equal(philox.uniform(philox.accept_words(3, 2, 12, 0)), a[2, 2])
