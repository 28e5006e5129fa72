"""GPU parity of the acceptance probability and accept-length law (specverify_accept_prob)
against the fp64 oracle, through the C ABI.

The normalisers fed to the entry point are the GPU step's own outputs (the
composition a caller runs); the oracle computes everything from the logits.
Bar: |d alpha| <= 5e-7 (float32 terms around per-lane references of each row,
float64 sums, plus the step's |d ln Z| <= ~1.4e-7; measured <= 1.7e-7),
|d P(n = m)| <= 1e-6; greedy rows exact.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import device_draft_verification_specverify_amd as sv
import oracle
import workloads
from gpu_helpers import device, logits_to_dev, to_dev

pytestmark = pytest.mark.gpu

ALPHA_TOL = 5e-7
LAW_TOL = 1e-6


def _run(w, target=None, draft=None):
    dev = device()
    t = logits_to_dev(w.target, w.dtype) if target is None else target
    d = logits_to_dev(w.draft, w.dtype) if draft is None else draft
    temp = to_dev(w.temperature)
    out = sv.specverify_step(t, d, to_dev(w.tokens), temp, w.seed, to_dev(w.pos0))
    lnz_d = torch.nan_to_num(out.lnZ_draft, nan=0.0)  # greedy rows: not read
    alpha, law = sv.specverify_accept_prob(t, d, temp, out.lnZ_target, lnz_d)
    torch.cuda.synchronize(dev)
    return alpha.cpu().numpy(), law.cpu().numpy()


def _compare(w, alpha, law, rows=None):
    sel = np.arange(w.B) if rows is None else np.asarray(rows)
    ref = oracle.acceptance_probability(w.target[sel], w.draft[sel], w.temperature[sel],
                                        dtype=w.dtype)
    ref_law = oracle.outcome_law(ref)
    a, lw = alpha[sel], law[sel]
    T = w.temperature[sel]
    greedy = T == 0
    assert np.array_equal(a[greedy], ref[greedy])
    assert np.array_equal(lw[greedy], ref_law[greedy])
    da = np.abs(a[~greedy] - ref[~greedy])
    dl = np.abs(lw[~greedy] - ref_law[~greedy])
    assert da.size == 0 or da.max() <= ALPHA_TOL, f"max |d alpha| = {da.max()}"
    assert dl.size == 0 or dl.max() <= LAW_TOL, f"max |d law| = {dl.max()}"
    np.testing.assert_allclose(law.sum(axis=-1), 1.0, atol=1e-12)
    stats = {"chains": int(a.shape[0] * a.shape[1]),
             "max_dalpha": float(da.max()) if da.size else 0.0,
             "max_dlaw": float(dl.max()) if dl.size else 0.0,
             "mean_alpha": float(np.nanmean(ref))}
    print(f"[parity] accept_prob {w.name}: {stats}", flush=True)
    return stats


@pytest.mark.parametrize("name,kw", [
    ("c1", {}), ("c2", {}), ("c3", dict(B=16)), ("c4", dict(B=32)), ("c5", dict(B=4)),
])
def test_accept_prob_matches_oracle(name, kw):
    w = workloads.make(name, **kw)
    print(f"[case] accept_prob {name} {kw}", flush=True)
    alpha, law = _run(w)
    _compare(w, alpha, law)


def test_accept_prob_c3_full():
    w = workloads.make("c3")
    print("[case] accept_prob c3 full B=64", flush=True)
    alpha, law = _run(w)
    _compare(w, alpha, law)


def test_accept_prob_c5_full_sampled_rows():
    w = workloads.make("c5")
    print("[case] accept_prob c5 full B=512 K=4, oracle on 6 rows", flush=True)
    alpha, law = _run(w)
    _compare(w, alpha, law, rows=[0, 1, 200, 301, 510, 511])
    assert np.all((alpha > 0) & (alpha < 1))


@pytest.mark.parametrize("V,gamma,K,B,dtype", [
    (1, 2, 1, 3, "bf16"), (7, 3, 2, 5, "f32"), (9, 4, 1, 6, "bf16"), (4097, 8, 1, 9, "bf16"),
    (8193, 2, 3, 5, "bf16"), (40001, 6, 1, 3, "f32"), (33000, 32, 2, 2, "bf16"),
])
def test_accept_prob_edge_shapes(V, gamma, K, B, dtype):
    print(f"[case] accept_prob edge V={V} gamma={gamma} K={K} B={B} {dtype}", flush=True)
    w = workloads.make("c4", B=B, V=V, gamma=gamma, K=K, dtype=dtype)
    alpha, law = _run(w)
    _compare(w, alpha, law)


def test_accept_prob_unaligned_rows_and_identical_drafts():
    # element loads (rows 2 bytes off alignment) and draft == target (alpha = 1)
    w = workloads.make("c2", B=3, V=1001)
    print("[case] accept_prob unaligned V=1001 bf16", flush=True)
    dev = device()
    raw_t = logits_to_dev(w.target, w.dtype)
    big = torch.zeros(raw_t.numel() + 1, dtype=raw_t.dtype, device=dev)
    big[1:] = raw_t.reshape(-1)
    t = big[1:].view(raw_t.shape)
    d = t[:, :-1].unsqueeze(1)                     # the target rows themselves, strided
    same = w.target[:, :-1][:, None].copy()
    w2 = workloads.Workload(name="same", B=w.B, K=1, gamma=w.gamma, V=w.V, dtype=w.dtype,
                            target=w.target, draft=same, tokens=w.tokens, temperature=w.temperature,
                            pos0=w.pos0, seed=w.seed)
    alpha, law = _run(w2, target=t, draft=d)
    np.testing.assert_allclose(alpha, 1.0, atol=ALPHA_TOL)
    _compare(w2, alpha, law)


def test_accept_prob_invalid_temperature_is_nan():
    w = workloads.make("c2", B=2, V=512)
    w.temperature[1] = -1.0
    dev = device()
    t, d = logits_to_dev(w.target, w.dtype), logits_to_dev(w.draft, w.dtype)
    lz_t = torch.zeros((w.B, w.gamma + 1), dtype=torch.float64, device=dev)
    lz_d = torch.zeros((w.B, 1, w.gamma), dtype=torch.float64, device=dev)
    alpha, law = sv.specverify_accept_prob(t, d, to_dev(w.temperature), lz_t, lz_d)
    a = alpha.cpu().numpy()
    assert np.isnan(a[1]).all() and not np.isnan(a[0]).any()
