"""GPU parity of the residual top-F candidates (specverify_residual_topf) and the cache
lookup (specverify_cache_lookup) against the fp64 oracle, through the C ABI.

Bar: every listed id is the oracle's id at that rank, or an id whose oracle
weight equals the oracle's weight at that rank within 2e-6 of the row's top
weight (float32 ranking swaps only near-equal weights); padding (-1) exactly
where the oracle's support ends, except for ids whose weight is that close to
0; ids distinct within an outcome; greedy rows exact. The lookup is integer
work on the GPU's own candidates and must match the oracle's lookup exactly.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import device_draft_verification_specverify_amd as sv
import oracle
import workloads
from gpu_helpers import device, logits_to_dev, to_dev
from oracle import speculation_cache as sc

pytestmark = pytest.mark.gpu

REL = 2e-6


def _run(w, fan, target=None, draft=None):
    dev = device()
    t = logits_to_dev(w.target, w.dtype) if target is None else target
    d = logits_to_dev(w.draft, w.dtype) if draft is None else draft
    temp = to_dev(w.temperature)
    out = sv.specverify_step(t, d, to_dev(w.tokens), temp, w.seed, to_dev(w.pos0))
    lnz_d = torch.nan_to_num(out.lnZ_draft, nan=0.0)
    cand, cw = sv.specverify_residual_topf(t, d, temp, out.lnZ_target, lnz_d, fan,
                                           want_weights=True)
    slot = sv.specverify_cache_lookup(cand, fan, out.accept_len, out.out_token)
    torch.cuda.synchronize(dev)
    return (cand.cpu().numpy(), cw.cpu().numpy(), slot.cpu().numpy(),
            out.accept_len.cpu().numpy(), out.out_token.cpu().numpy())


def _compare(w, fan, cand, slot, n, y, rows=None):
    sel = np.arange(w.B) if rows is None else np.asarray(rows)
    ref, _ = sc.residual_topf(w.target[sel], w.draft[sel], w.temperature[sel], fan, dtype=w.dtype)
    wts = sc.outcome_weights(w.target[sel], w.draft[sel], w.temperature[sel], dtype=w.dtype)
    c = cand[sel]
    T = w.temperature[sel]
    greedy = T == 0
    assert np.array_equal(c[greedy], ref[greedy]), "greedy rows differ"
    swapped = 0
    offs = np.concatenate([[0], np.cumsum(fan)])
    for bi in range(c.shape[0]):
        if greedy[bi]:
            continue
        for k in range(c.shape[1]):
            for j in range(len(fan)):
                gl = c[bi, k, offs[j]:offs[j + 1]]
                rl = ref[bi, k, offs[j]:offs[j + 1]]
                if np.array_equal(gl, rl):
                    continue
                wj = wts[bi, k, j]
                fin = wj[np.isfinite(wj)]
                top = float(fin.max()) if fin.size else 0.0   # no support at all: 0
                listed = gl[gl >= 0]
                assert len(set(listed.tolist())) == listed.size, "repeated id"
                for i in range(len(gl)):
                    if gl[i] == rl[i]:
                        continue
                    want = wj[rl[i]] if rl[i] >= 0 else 0.0
                    got = wj[gl[i]] if gl[i] >= 0 else 0.0
                    got = 0.0 if got == -np.inf else got
                    want = 0.0 if want == -np.inf else want
                    assert abs(got - want) <= REL * top, (bi, k, j, i, gl[i], rl[i], got, want)
                    swapped += 1
    want_slot = sc.cache_lookup(c, fan, n[sel], y[sel])
    assert np.array_equal(slot[sel], want_slot)
    stats = {"chains": int(c.shape[0] * c.shape[1]), "near_tie_swaps": swapped,
             "hit_rate": float(np.mean(slot[sel] >= 0))}
    print(f"[parity] topf {w.name} fan={list(fan)}: {stats}", flush=True)
    return stats


@pytest.mark.parametrize("name,kw,total,ratio", [
    ("c1", {}, 20, 0.6), ("c2", {}, 24, 0.7), ("c3", dict(B=16), 36, 0.6),
    ("c4", dict(B=32), 20, 0.5), ("c5", dict(B=4), 45, 0.65),
])
def test_topf_matches_oracle(name, kw, total, ratio):
    w = workloads.make(name, **kw)
    fan = sv.geometric_fanout(w.gamma, total, ratio)
    print(f"[case] topf {name} {kw} fan={fan}", flush=True)
    cand, cw, slot, n, y = _run(w, fan)
    _compare(w, fan, cand, slot, n, y)
    assert np.all(cw[cand < 0] == -np.inf)


def test_topf_c3_full_and_large_fanout():
    w = workloads.make("c3")
    fan = [64, 48, 32, 16, 8, 4, 2, 1, 64]
    print(f"[case] topf c3 full fan={fan}", flush=True)
    cand, _, slot, n, y = _run(w, fan)
    _compare(w, fan, cand, slot, n, y, rows=np.arange(0, 64, 3))


@pytest.mark.parametrize("V,gamma,K,B,dtype,fan", [
    (1, 2, 1, 3, "bf16", [2, 1, 1]), (7, 3, 2, 5, "f32", [8, 4, 2, 8]),
    (9, 4, 1, 6, "bf16", [3, 3, 3, 3, 3]), (4097, 8, 1, 4, "bf16", [64] * 9),
    (8193, 2, 3, 5, "bf16", [5, 0, 7]), (40001, 6, 1, 3, "f32", [1] * 7),
    (33000, 32, 2, 2, "bf16", [2] * 33),
])
def test_topf_edge_shapes(V, gamma, K, B, dtype, fan):
    print(f"[case] topf edge V={V} gamma={gamma} K={K} B={B} {dtype} fan={fan}", flush=True)
    w = workloads.make("c4", B=B, V=V, gamma=gamma, K=K, dtype=dtype)
    cand, _, slot, n, y = _run(w, fan)
    _compare(w, fan, cand, slot, n, y)


def test_topf_greedy_ties_and_invalid_temperature():
    # bf16 rows with many equal logits: greedy candidates follow the lowest-id rule exactly
    w = workloads.make("c4", B=4, V=3000, temps=("const", 0.0))
    w.target[:] = (w.target & np.uint16(0xFFC0))      # coarse bf16 values: many exact ties
    fan = [16, 8, 8, 4, 16]
    cand, _, slot, n, y = _run(w, fan)
    _compare(w, fan, cand, slot, n, y)
    w2 = workloads.make("c2", B=2, V=512)
    w2.temperature[1] = -1.0
    dev = device()
    t, d = logits_to_dev(w2.target, w2.dtype), logits_to_dev(w2.draft, w2.dtype)
    lz_t = torch.zeros((w2.B, w2.gamma + 1), dtype=torch.float64, device=dev)
    lz_d = torch.zeros((w2.B, 1, w2.gamma), dtype=torch.float64, device=dev)
    cand2, _ = sv.specverify_residual_topf(t, d, to_dev(w2.temperature), lz_t, lz_d, [2] * 6)
    c2 = cand2.cpu().numpy()
    assert np.all(c2[1] == -1) and np.all(c2[0] >= 0)


def test_topf_large_grid_takes_the_narrow_sample():
    # 512 x 6 = 3072 rows, more than 8 per CU: the launch samples 8 passes (not the
    # 16 of grids with 1 to 8 rows per CU, such as the full C3 case above)
    w = workloads.make("c2", B=512, V=8000)
    fan = sv.geometric_fanout(w.gamma, 24, 0.7)
    print(f"[case] topf large grid B={w.B} V={w.V} fan={fan}", flush=True)
    cand, _, slot, n, y = _run(w, fan)
    _compare(w, fan, cand, slot, n, y, rows=np.arange(0, 512, 16))


def test_topf_massive_ties_cut_every_wavefront_region():
    # z_t = 0 everywhere and z_d = -10 except on every 7th id (+10, no residual mass
    # there): the residual weight is the same float on 6 ids of 7 and the bonus
    # weight on every id, so each wavefront admits ~440 ids a step and cuts its
    # region every step; the best F are then exactly the lowest ids
    w = workloads.make("c3", B=2, V=40000, gamma=2, temps=("const", 1.0))
    w.target[:] = np.uint16(0x0000)
    w.draft[:] = np.uint16(0xC120)
    w.draft[..., ::7] = np.uint16(0x4120)
    fan = [64, 64, 64]
    print(f"[case] topf massive ties V={w.V} fan={fan}", flush=True)
    cand, _, slot, n, y = _run(w, fan)
    ref, _ = sc.residual_topf(w.target, w.draft, w.temperature, fan, dtype=w.dtype)
    want_res = np.array([v for v in range(200) if v % 7][:64])
    assert np.array_equal(ref[0, 0, :64], want_res)          # the reading the oracle fixes
    assert np.array_equal(ref[0, 0, 128:], np.arange(64))
    assert np.array_equal(cand, ref)
    _compare(w, fan, cand, slot, n, y)


def test_hit_rate_tracks_the_law_on_the_gpu():
    # many replicate chains of one batch row: the GPU cache hit rate over the GPU step's
    # outcomes matches the rate the oracle predicts from alpha and the residual masses
    base = workloads.make("c2", B=1, V=64)
    reps = 4096
    rng = np.random.default_rng(3)
    from scipy.special import softmax
    zt = oracle.decode_logits(base.target[0], "bf16")
    zd = oracle.decode_logits(base.draft[0, 0], "bf16")
    T = float(base.temperature[0])
    q = softmax(zd / T, axis=-1)
    toks = np.stack([rng.choice(base.V, size=reps, p=q[j]) for j in range(base.gamma)], axis=1)
    w = workloads.Workload(name="reps", B=reps, K=1, gamma=base.gamma, V=base.V, dtype="bf16",
                           target=np.ascontiguousarray(np.broadcast_to(base.target, (reps,) + base.target.shape[1:])),
                           draft=np.ascontiguousarray(np.broadcast_to(base.draft, (reps,) + base.draft.shape[1:])),
                           tokens=toks[:, None, :].astype(np.int32),
                           temperature=np.full(reps, base.temperature[0], np.float32),
                           pos0=np.arange(reps, dtype=np.int64), seed=base.seed)
    fan = sv.geometric_fanout(w.gamma, 18, 0.6)
    cand, _, slot, n, y = _run(w, fan)
    hit = float(np.mean(slot >= 0))
    ref, _ = sc.residual_topf(base.target, base.draft, base.temperature, fan, dtype="bf16")
    alpha = oracle.acceptance_probability(base.target, base.draft, base.temperature, dtype="bf16")
    law = oracle.outcome_law(alpha)[0, 0]
    wts = sc.outcome_weights(base.target, base.draft, base.temperature, dtype="bf16")[0, 0]
    offs = np.concatenate([[0], np.cumsum(fan)])
    want = 0.0
    for j in range(w.gamma + 1):
        wj = np.where(np.isfinite(wts[j]), wts[j], 0.0)
        ids = ref[0, 0, offs[j]:offs[j + 1]]
        want += law[j] * wj[ids[ids >= 0]].sum() / wj.sum()
    print(f"[parity] topf hit rate gpu {hit:.4f} predicted {want:.4f}", flush=True)
    assert abs(hit - want) < 5 * np.sqrt(want * (1 - want) / reps)
