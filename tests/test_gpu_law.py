"""Distribution gate on the HIP path itself: the fused step run on 10^6 replicate
chains against the exact law of the emitted tokens.

FlashSpec (technical summary, section 3 "Correctness and testing") gates the
verifier's outputs with a distribution-equivalence test at alpha = 0.01 and
stresses that large samples are needed to see subtle shifts. Here the HIP step
verifies 10^6 chains that share one target and one draft context (stride-0
rows), each with its own draft tokens x_j ~ q_j; the outcomes (n, x_<n, y)
must follow

    P(n = k, x_<k, y) = prod_{j<k} min(p_j, q_j)(x_j) * [max(p_k - q_k, 0)(y) or p_gamma(y)]

by a chi-square test at alpha = 0.01 (cells with expected count < 5 merged),
and every emitted token must be distributed as the target alone would draw it.
The 10^6 chains also take the library's path for more than 65,536 chains.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch
from scipy.special import softmax

import device_draft_verification_specverify_amd as sv
from gpu_helpers import device, to_dev
from test_oracle_law import ALPHA, G, N_REPLICATES, SEED, T32, V, _cell_index, _chi2_pvalue, \
    _exact_law

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gpu_replicates():
    rng = np.random.default_rng(12345)
    zt = rng.normal(0, 1.5, size=(G + 1, V)).astype(np.float32)
    zd = (zt[:G] + rng.normal(0, 1.0, size=(G, V))).astype(np.float32)
    p = softmax(zt.astype(np.float64) / T32, axis=1)
    q = softmax(zd.astype(np.float64) / T32, axis=1)
    N = N_REPLICATES
    trng = np.random.default_rng(778)
    toks = np.stack([trng.choice(V, size=N, p=q[j]) for j in range(G)], axis=1).astype(np.int32)
    print(f"[case] gpu law: {N} chains, V={V}, gamma={G}, T={T32}", flush=True)
    dev = device()
    target = to_dev(zt)[None].expand(N, G + 1, V)          # stride 0 over the batch
    draft = to_dev(zd)[None, None].expand(N, 1, G, V)
    out = sv.specverify_step(target, draft, to_dev(toks[:, None, :]),
                             torch.full((N,), T32, dtype=torch.float32, device=dev), SEED, None)
    torch.cuda.synchronize(dev)
    n = out.accept_len[:, 0].cpu().numpy().astype(np.int64)
    y = out.out_token[:, 0].cpu().numpy().astype(np.int64)
    assert int(out.device_error.item()) == 0
    return n, toks.astype(np.int64), y, p, q


def test_gpu_outcome_law_chi2_gate(gpu_replicates):
    n, toks, y, p, q = gpu_replicates
    assert np.all((n >= 0) & (n <= G)) and np.all((y >= 0) & (y < V))
    law = _exact_law(p, q)
    counts = np.bincount(_cell_index(n, toks, y), minlength=law.size)
    assert counts.size == law.size
    pval = _chi2_pvalue(counts, law, n.size)
    print(f"[parity] gpu law chi2 p = {pval:.3f}", flush=True)
    assert pval >= ALPHA, pval


def test_gpu_emitted_tokens_follow_the_target(gpu_replicates):
    n, toks, y, p, q = gpu_replicates
    first = np.where(n >= 1, toks[:, 0], y)
    assert _chi2_pvalue(np.bincount(first, minlength=V), p[0], n.size) >= ALPHA
    sel = n >= 1
    second = np.where(n[sel] >= 2, toks[sel, 1], y[sel])
    assert _chi2_pvalue(np.bincount(second, minlength=V), p[1], int(sel.sum())) >= ALPHA
    sel = n == G
    assert _chi2_pvalue(np.bincount(y[sel], minlength=V), p[G], int(sel.sum())) >= ALPHA
    # a rejected draft token is never the correction (it lies outside the residual's support)
    rej = n < G
    assert not np.any(y[rej] == toks[rej, n[rej]])
