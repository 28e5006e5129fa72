"""Pins for the oracle's temperature + normaliser + gather steps (CPU only).

Each test checks the oracle against something other than itself: closed forms,
library routines the oracle does not call (scipy's logsumexp, torch's
log_softmax and bfloat16 conversion), hand-derived fixtures and exact
metamorphic relations.
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax

import oracle
from oracle import specverify as sv


@pytest.mark.parametrize("T", [0.1, 0.7, 1.0, 3.0])
@pytest.mark.parametrize("V", [1, 2, 7, 1000])
def test_constant_row_closed_form(T, V):
    c = 1.75
    lnz, am = sv.normalize_rows(np.full((3, V), c), np.full(3, T))
    assert np.allclose(lnz, np.log(V) + c / T, rtol=0, atol=1e-12)
    assert np.all(am == 0)


@pytest.mark.parametrize("T", [0.25, 1.0, 2.0])
def test_one_hot_and_two_entry_closed_forms(T):
    V, a = 50, 3.0
    z = np.zeros((V, V))
    z[np.arange(V), np.arange(V)] = a
    lnz, am = sv.normalize_rows(z, np.full(V, T))
    assert np.allclose(lnz, np.log(np.exp(a / T) + V - 1), rtol=1e-14)
    assert np.array_equal(am, np.arange(V))
    # V = 2: ln Z = b/T + softplus((a - b)/T)
    x = np.array([[0.3, -1.2], [5.0, 5.5], [-40.0, 40.0]])
    lnz2, _ = sv.normalize_rows(x, np.full(3, T))
    want = x[:, 1] / T + np.log1p(np.exp((x[:, 0] - x[:, 1]) / T))
    assert np.allclose(lnz2, want, rtol=1e-14)


def test_against_scipy_logsumexp_and_torch_log_softmax():
    rng = np.random.default_rng(7)
    z = rng.normal(0, 3, size=(6, 4, 3001))
    T = np.array([0.1, 0.4, 0.7, 1.0, 1.3, 5.0])
    lnz, _ = sv.normalize_rows(z, T[:, None])
    ref = logsumexp(z / T[:, None, None], axis=-1)
    assert np.allclose(lnz, ref, rtol=1e-13, atol=1e-12)
    # gathered log-probs via the full verification on a K=1 chain
    tok = rng.integers(0, 3001, size=(6, 1, 3))
    out = oracle.verify(z[:, :4], z[:, None, :3] + 0.5, tok, T, seed=5, pos0=np.zeros(6, int))
    Tt = torch.tensor(np.float32(T).astype(np.float64))
    lsm_t = torch.log_softmax(torch.tensor(z[:, :4]) / Tt[:, None, None], dim=-1).numpy()
    lsm_d = torch.log_softmax(torch.tensor(z[:, :3] + 0.5) / Tt[:, None, None], dim=-1).numpy()
    bb = np.arange(6)[:, None]
    jj = np.arange(3)[None, :]
    assert np.allclose(out["logp"][:, 0], lsm_t[bb, jj, tok[:, 0]], atol=1e-12)
    assert np.allclose(out["logq"][:, 0], lsm_d[bb, jj, tok[:, 0]], atol=1e-12)


def test_temperature_before_log_softmax_fixture(golden):
    fx = golden("temperature_order.json")
    z = np.array([fx["logits"]])
    lnz, _ = sv.normalize_rows(z, np.array([fx["T"]]))
    assert np.isclose(lnz[0], fx["lnZ"], rtol=1e-14)
    p = np.exp(z[0] / fx["T"] - lnz[0])
    assert np.allclose(p, fx["p"], rtol=1e-13)
    # the wrong order (temperature after the log-softmax) does not give a distribution
    wrong = np.exp((z[0] - logsumexp(z[0])) / fx["T"])
    assert np.isclose(wrong.sum(), fx["wrong_order_total_mass"], rtol=1e-13)


def test_greedy_rows_max_and_lowest_argmax(golden):
    fx = golden("greedy_ties.json")
    z = np.array([fx["target_row"]])
    lnz, am = sv.normalize_rows(z, np.array([0.0]))
    assert lnz[0] == max(fx["target_row"]) and am[0] == fx["argmax"]
    rng = np.random.default_rng(3)
    zz = rng.integers(-3, 3, size=(200, 64)).astype(np.float64)     # many ties
    lnz, am = sv.normalize_rows(zz, np.zeros(200))
    assert np.array_equal(am, np.argmax(zz, axis=1))
    first = np.array([np.flatnonzero(r == r.max())[0] for r in zz])
    assert np.array_equal(am, first) and np.array_equal(lnz, zz.max(axis=1))


def test_masked_tokens_and_all_masked_rows():
    z = np.array([[0.0, -np.inf, np.log(3.0), -np.inf], [-np.inf] * 4])
    lnz, _ = sv.normalize_rows(z, np.array([1.0, 1.0]))
    assert np.isclose(lnz[0], np.log(4.0)) and np.isneginf(lnz[1])
    lnz_bad, _ = sv.normalize_rows(z[:1], np.array([-1.0]))
    assert np.isnan(lnz_bad[0])


def test_power_of_two_scaling_is_bit_exact():
    rng = np.random.default_rng(11)
    z = rng.normal(0, 2, size=(4, 2, 513))
    T = np.array([0.1, 0.7, 1.0, 3.0])
    base = sv.normalize_rows(z, T[:, None])[0]
    for k in (-3, 2, 5):
        s = 2.0 ** k
        assert np.array_equal(sv.normalize_rows(z * s, T[:, None] * s)[0], base)


def test_shift_invariance():
    rng = np.random.default_rng(12)
    z = rng.normal(0, 2, size=(3, 999))
    T = np.array([0.3, 1.0, 2.5])
    c = 17.25
    a = sv.normalize_rows(z, T)[0]
    b = sv.normalize_rows(z + c, T)[0]
    assert np.allclose(b - a, c / T, rtol=0, atol=1e-12)


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2 ** 16, size=100_000, dtype=np.uint64).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]                       # finite values only
    ours = sv.decode_logits(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_softmax_probabilities_sum_to_one():
    rng = np.random.default_rng(9)
    z = rng.normal(0, 4, size=(5, 2000))
    T = np.array([0.1, 0.5, 1, 2, 8.0])
    lnz, _ = sv.normalize_rows(z, T)
    p = np.exp(z / T[:, None] - lnz[:, None])
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-12)
    assert np.allclose(p, softmax(z / T[:, None], axis=1), atol=1e-15, rtol=1e-12)
