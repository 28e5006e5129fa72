"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar: accept lengths and emitted tokens bit-exact except chains the oracle flags
as within 1e-6 of a decision threshold; ln p / ln q within 1e-4 absolute;
normalisers within 1e-5 relative (|d ln Z| <= 1e-5); greedy rows exact.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import device_draft_verification_specverify_amd as sv
import oracle
import workloads
from gpu_helpers import LNZ_TOL, compare_step, device, logits_to_dev, step_on_gpu, to_dev

pytestmark = pytest.mark.gpu


def _ref(w, rows=None):
    if rows is None:
        return oracle.verify(w.target, w.draft, w.tokens, w.temperature, w.seed, w.pos0,
                             dtype=w.dtype)
    rows = np.asarray(rows)
    return oracle.verify(w.target[rows], w.draft[rows], w.tokens[rows], w.temperature[rows],
                         w.seed, w.pos0[rows], batch_index=rows, dtype=w.dtype)


def _report(name, stats):
    print(f"[parity] {name}: {stats}", flush=True)


@pytest.mark.parametrize("name,kw", [
    ("c1", {}), ("c2", {}), ("c3", dict(B=16)), ("c4", dict(B=32)), ("c5", dict(B=4)),
])
def test_step_matches_oracle_reduced_batches(name, kw):
    w = workloads.make(name, **kw)
    print(f"[case] {name} {kw}", flush=True)
    gpu = step_on_gpu(w)
    _report(name, compare_step(gpu, _ref(w), w.temperature))
    assert int(gpu["device_error"][0]) == 0


def test_step_matches_oracle_c3_full():
    w = workloads.make("c3")
    print("[case] c3 full B=64", flush=True)
    gpu = step_on_gpu(w)
    _report("c3", compare_step(gpu, _ref(w), w.temperature))


def test_step_matches_oracle_c4_full_sampled_rows():
    w = workloads.make("c4")
    print("[case] c4 full B=256, oracle on 64 rows", flush=True)
    gpu = step_on_gpu(w)
    rows = np.concatenate([np.arange(16), np.random.default_rng(4).choice(np.arange(16, 256), 48,
                                                                          replace=False)])
    _report("c4", compare_step(gpu, _ref(w, rows), w.temperature, rows))


def test_step_matches_oracle_c5_full_sampled_rows():
    w = workloads.make("c5")
    rows = np.unique(np.concatenate([[0, 1, 77, 128, 255, 256, 300, 411, 510, 511],
                                     np.random.default_rng(5).choice(512, 22, replace=False)]))
    print(f"[case] c5 full B=512 K=4, oracle on {rows.size} rows ({4 * rows.size} chains)",
          flush=True)
    gpu = step_on_gpu(w)
    _report("c5", compare_step(gpu, _ref(w, rows), w.temperature, rows))
    # properties at every chain: lengths in range, corrections differ from the rejected draft
    n, y = gpu["accept_len"], gpu["out_token"]
    assert np.all((n >= 0) & (n <= w.gamma)) and np.all((y >= 0) & (y < w.V))
    bb, kk = np.nonzero(n < w.gamma)
    assert np.all(y[bb, kk] != w.tokens[bb, kk, n[bb, kk]])


@pytest.mark.parametrize("V,gamma,K,B,dtype", [
    (1, 2, 1, 3, "bf16"), (7, 3, 2, 5, "f32"), (8, 1, 1, 4, "bf16"), (9, 4, 1, 6, "bf16"),
    (1000, 5, 1, 7, "f32"), (4097, 8, 1, 9, "bf16"), (8193, 2, 3, 5, "bf16"),
    (40001, 6, 1, 3, "f32"), (33000, 32, 2, 2, "bf16"), (5000, 16, 4, 3, "bf16"),
])
def test_edge_shapes(V, gamma, K, B, dtype):
    print(f"[case] edge V={V} gamma={gamma} K={K} B={B} {dtype}", flush=True)
    w = workloads.make("c3", B=B, V=V, gamma=gamma, K=K, dtype=dtype,
                       temps=("choice", (0.0, 0.3, 1.0, 2.5)))
    _report(f"edge V={V}", compare_step(step_on_gpu(w), _ref(w), w.temperature))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_unaligned_rows_take_the_element_path(dtype):
    w = workloads.make("c2", B=5, V=3001, dtype=dtype)
    print(f"[case] unaligned {dtype}", flush=True)
    # views whose rows start one element past a 16-byte boundary
    tpad = np.zeros(w.target.shape[:-1] + (w.V + 1,), dtype=w.target.dtype)
    dpad = np.zeros(w.draft.shape[:-1] + (w.V + 1,), dtype=w.draft.dtype)
    tpad[..., 1:] = w.target
    dpad[..., 1:] = w.draft
    t = logits_to_dev(tpad, w.dtype)[..., 1:]
    d = logits_to_dev(dpad, w.dtype)[..., 1:]
    assert t.data_ptr() % 16 != 0
    _report("unaligned", compare_step(step_on_gpu(w, target=t, draft=d), _ref(w), w.temperature))


def test_broadcast_target_and_draft_rows():
    w = workloads.make("c3", B=1, V=6000)
    B = 24
    print("[case] broadcast stride 0", flush=True)
    tb = np.broadcast_to(w.target, (B,) + w.target.shape[1:])
    db = np.broadcast_to(w.draft, (B,) + w.draft.shape[1:])
    rng = np.random.default_rng(1)
    tokens = rng.integers(0, w.V, size=(B, 1, w.gamma)).astype(np.int32)
    temps = np.full(B, w.temperature[0], dtype=np.float32)
    pos0 = np.arange(B, dtype=np.int64) * 3
    w2 = workloads.Workload("bcast", B, 1, w.gamma, w.V, w.dtype, np.ascontiguousarray(tb),
                            np.ascontiguousarray(db), tokens, temps, pos0, w.seed)
    t = logits_to_dev(w.target, w.dtype).expand(B, -1, -1)
    d = logits_to_dev(w.draft, w.dtype).expand(B, -1, -1, -1)
    assert t.stride(0) == 0 and d.stride(0) == 0
    g_b = step_on_gpu(w2, target=t, draft=d)
    g_c = step_on_gpu(w2)
    for k in ("accept_len", "out_token", "logp", "logq", "lnZ_target"):
        assert np.array_equal(g_b[k], g_c[k]), k
    _report("broadcast", compare_step(g_b, _ref(w2), temps))


def test_reruns_are_bit_identical():
    w = workloads.make("c3", B=12)
    print("[case] determinism", flush=True)
    a = step_on_gpu(w)
    b = step_on_gpu(w)
    for k, v in a.items():
        if v is not None:
            assert np.array_equal(v, b[k], equal_nan=True), k


def test_input_errors_set_bits_and_poison_only_their_chains():
    w = workloads.make("c3", B=8, V=2000, temps=("const", 0.7))
    print("[case] error paths", flush=True)
    w.tokens[1, 0, 2] = w.V               # out of range
    w.tokens[2, 0, 0] = -5
    w.temperature[3] = -1.0
    w.temperature[4] = np.nan
    if w.dtype == "bf16":
        w.target[5, 3, :] = 0xFF80        # -inf row
    gpu = step_on_gpu(w)
    ref = _ref(w)
    assert np.array_equal(gpu["accept_len"], ref["accept_len"])
    assert int(gpu["device_error"][0]) == ref["error"] == (1 | 2 | 4)
    for b in (1, 2, 3, 4, 5):
        assert gpu["accept_len"][b, 0] == -1 and gpu["out_token"][b, 0] == -1
    good = np.array([0, 6, 7])
    compare_step({k: (v[good] if k not in ("device_error",) and v is not None else v)
                  for k, v in gpu.items()},
                 {k: (v[good] if isinstance(v, np.ndarray) and v.ndim >= 1 else v)
                  for k, v in ref.items()}, w.temperature[good])


def test_normalize_entry_point():
    rng = np.random.default_rng(2)
    for V, dt in ((1, "f32"), (300, "bf16"), (128256, "bf16"), (32001, "f32")):
        print(f"[case] normalize V={V} {dt}", flush=True)
        B, P = 5, 3
        z = rng.normal(0, 3, size=(B, P, V)).astype(np.float32)
        z[0, 0, : V // 2] = -np.inf
        raw = workloads.round_to_bf16_bits(z) if dt == "bf16" else z
        T = np.array([0.0, 0.1, 0.7, 1.0, 3.0], dtype=np.float32)
        lnz, am = sv.specverify_normalize(logits_to_dev(raw, dt), to_dev(T), want_argmax=True)
        torch.cuda.synchronize()
        zz = oracle.decode_logits(raw, dt)
        rl, ra = oracle.normalize_rows(zz, T[:, None])
        lnz, am = lnz.cpu().numpy(), am.cpu().numpy()
        assert np.array_equal(am, ra)
        assert np.array_equal(lnz[0], rl[0])                       # greedy row: the raw max
        assert np.all(np.abs(lnz[1:] - rl[1:]) <= 1e-5), np.abs(lnz[1:] - rl[1:]).max()


@pytest.mark.parametrize("name,kw", [("c2", {}), ("c3", dict(B=8)), ("c4", dict(B=6)),
                                     ("c2", dict(B=700))])
def test_normalize_and_step_give_the_same_normalisers(name, kw):
    # B=700 at V=32000: 2800 draw workgroups, more than fit at once, so the step takes
    # the separate accept launch (the same fold order as the fused prologue)
    # both fold a row's chunk partials with the same lanes in the same order, so a
    # caller gets the same ln Z bits from either entry point
    w = workloads.make(name, **kw)
    print(f"[case] normalize vs step {name} {kw}", flush=True)
    t, d = logits_to_dev(w.target, w.dtype), logits_to_dev(w.draft, w.dtype)
    temp = to_dev(w.temperature)
    out = sv.specverify_step(t, d, to_dev(w.tokens), temp, w.seed, to_dev(w.pos0))
    lz_t, am = sv.specverify_normalize(t, temp, want_argmax=True)
    lz_d, _ = sv.specverify_normalize(d[:, 0], temp)
    torch.cuda.synchronize()
    assert torch.equal(lz_t, out.lnZ_target)
    sampled = torch.from_numpy(w.temperature > 0).to(t.device)
    assert torch.equal(lz_d[sampled], out.lnZ_draft[:, 0][sampled])
    want = oracle.normalize_rows(oracle.decode_logits(w.target, w.dtype), w.temperature[:, None])[1]
    assert np.array_equal(am.cpu().numpy(), want)


def test_accept_entry_point_reproduces_the_oracle_exactly():
    rng = np.random.default_rng(3)
    for B, K, g in ((256, 1, 4), (7, 4, 8), (3, 2, 32), (1, 1, 1)):
        print(f"[case] accept B={B} K={K} gamma={g}", flush=True)
        lp = rng.normal(-2, 1, size=(B, K, g)).astype(np.float32)
        lq = (lp + rng.normal(0, 0.7, size=lp.shape)).astype(np.float32)
        lp[0, 0, 0] = -np.inf                                       # greedy-style reject
        lq[-1, -1, -1] = -np.inf
        pos0 = rng.integers(0, 1 << 40, size=B).astype(np.int64)
        n, bits = sv.specverify_accept(to_dev(lp), to_dev(lq), 987654321, to_dev(pos0),
                                       want_bits=True)
        torch.cuda.synchronize()
        rn, rbits, _ = oracle.accept_from_logprobs(lp, lq, 987654321, pos0)
        assert np.array_equal(n.cpu().numpy(), rn)
        assert np.array_equal(bits.cpu().numpy().view(np.uint32), rbits)


def test_residual_entry_point_at_every_accept_length():
    w = workloads.make("c3", B=6, V=20000, temps=("choice", (0.0, 0.4, 1.0)))
    print("[case] residual entry point", flush=True)
    zt = oracle.decode_logits(w.target, w.dtype)
    zd = oracle.decode_logits(w.draft, w.dtype)
    ref = oracle.verify(zt, zd, w.tokens, w.temperature, w.seed, w.pos0)
    chain_rows = np.arange(w.B)[:, None]
    for n in range(w.gamma + 1):
        nn = np.full((w.B, 1), n, dtype=np.int64)
        tok, flag, _ = oracle.specverify.sample_tokens(
            zt, zd, w.temperature.astype(np.float64), ref["lnZ_target"],
            np.nan_to_num(ref["lnZ_draft"]), ref["argmax_target"], nn, w.seed, w.pos0, chain_rows)
        out = sv.specverify_residual_sample(
            logits_to_dev(w.target, w.dtype), logits_to_dev(w.draft, w.dtype), to_dev(w.temperature),
            to_dev(ref["lnZ_target"]), to_dev(np.nan_to_num(ref["lnZ_draft"])),
            to_dev(ref["argmax_target"].astype(np.int32)), to_dev(nn.astype(np.int32)), w.seed,
            to_dev(w.pos0))
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got[~flag], tok[~flag]), (n, got.ravel(), tok.ravel())


@pytest.mark.parametrize("B,K,gamma,V,dtype", [
    (16400, 1, 1, 40, "f32"),     # past the sampled-row table: draft rows of every batch row streamed
    (13200, 5, 1, 24, "bf16"),    # 66000 chains
])
def test_large_batches(B, K, gamma, V, dtype):
    print(f"[case] large batch B={B} K={K} gamma={gamma} V={V} {dtype}", flush=True)
    w = workloads.make("c3", B=B, V=V, gamma=gamma, K=K, dtype=dtype,
                       temps=("choice", (0.0, 0.5, 1.0)))
    gpu = step_on_gpu(w)
    rows = np.concatenate([np.arange(20), np.random.default_rng(5).choice(np.arange(20, B), 40,
                                                                          replace=False)])
    _report("large batch", compare_step(gpu, _ref(w, rows), w.temperature, rows))
    assert int(gpu["device_error"][0]) == 0


def test_workspace_reused_across_shapes_and_calls():
    """One workspace serves calls of different sizes and repeated calls."""
    shapes = [dict(B=8, V=5000, dtype="bf16"), dict(B=3, V=40000, dtype="f32", K=2),
              dict(B=8, V=5000, dtype="bf16"), dict(B=33, V=777, gamma=3, dtype="f32")]
    ws_bytes = max(sv.workspace_size(s["B"], s.get("K", 1), s.get("gamma", 8), s["V"],
                                     sv.SV_BF16 if s["dtype"] == "bf16" else sv.SV_F32)
                   for s in shapes)
    ws = torch.full((ws_bytes,), 0xFF, dtype=torch.uint8, device=device())  # any contents
    for i, s in enumerate(shapes):
        print(f"[case] shared workspace call {i}: {s}", flush=True)
        w = workloads.make("c3", seed=i, temps=("choice", (0.0, 0.3, 1.0)), **s)
        if i == 2:  # random bytes left by some other user of the memory
            gen = torch.Generator(device=device()).manual_seed(11)
            ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device=device(),
                                   generator=gen))
        shared = step_on_gpu(w, ws=ws)
        fresh = step_on_gpu(w)
        for k, v in fresh.items():
            if v is not None:
                assert np.array_equal(v, shared[k], equal_nan=True), (i, k)
        assert int(shared["device_error"][0]) == 0
        _report(f"shared ws {i}", compare_step(shared, _ref(w), w.temperature))
    # one plan called repeatedly on one stream
    w = workloads.make("c3", B=16, V=9000)
    plan = sv.StepPlan(logits_to_dev(w.target, w.dtype), logits_to_dev(w.draft, w.dtype),
                       to_dev(w.tokens), to_dev(w.temperature), w.seed, to_dev(w.pos0))
    first = None
    for _ in range(6):
        out = plan()
        torch.cuda.synchronize()
        cur = (out.accept_len.cpu().numpy().copy(), out.out_token.cpu().numpy().copy())
        first = first or cur
        assert np.array_equal(cur[0], first[0]) and np.array_equal(cur[1], first[1])
    assert int(plan.out.device_error.item()) == 0


def test_bandit_loop_over_draft_models_on_the_gpu():
    # three draft models of the same target (noise 0.3, 1.0, 2.5): a UCB1 loop of GPU
    # steps, rewarded with each step's accepted fraction, settles on the closest draft
    import workloads.synth as synth
    print("[case] bandit loop, 3 draft models, 60 steps", flush=True)
    base = workloads.make("c2", B=8, V=4000)
    rng = np.random.default_rng(0)
    zt = oracle.decode_logits(base.target, "bf16")
    dev = device()
    target = logits_to_dev(base.target, "bf16")
    temp = to_dev(base.temperature)
    models = []
    for sigma in (0.3, 1.0, 2.5):
        zd = zt[:, None, :-1] + rng.normal(0, sigma, size=base.draft.shape)
        models.append(logits_to_dev(synth._store(zd, "bf16"), "bf16"))
    bandit = sv.Bandit(3, sv.BANDIT_UCB1)
    picks, rewards = [], []
    for step in range(60):
        arm = bandit.select()
        draft = models[arm]
        # draft tokens: the draft model's own argmax, so every arm proposes its best guess
        toks = draft.float().argmax(dim=-1).to(torch.int32).contiguous()
        out = sv.specverify_step(target, draft, toks, temp, 1000 + step, to_dev(base.pos0))
        reward = sv.step_reward(out.accept_len, base.gamma)
        bandit.update(arm, reward)
        picks.append(arm)
        rewards.append(reward)
    counts = np.bincount(picks, minlength=3)
    print(f"[parity] bandit picks {counts.tolist()}", flush=True)
    assert counts[0] > counts[1] and counts[0] > counts[2]
    # the oracle's selector, fed the same rewards, picks the same arm at every step
    from oracle import bandit as bd
    ora = bd.Bandit(3, bd.UCB1)
    for step, (arm, reward) in enumerate(zip(picks, rewards)):
        assert ora.select() == arm, step
        ora.update(arm, reward)


def test_branch_prune_matches_the_oracle():
    # the pages give no rule (parity unpinned to them); the GPU must reproduce the
    # oracle's reading exactly: float64 running sums in order, integer ranks
    from oracle import branch_pruning as bp
    rng = np.random.default_rng(12)
    for B, K, g, tau, keep in ((37, 4, 8, 0.05, 2), (300, 8, 8, 0.2, 3), (5, 2, 32, 1e-3, 1),
                               (9, 16, 4, 0.5, 16), (3, 3, 3, 0.9, 0)):
        logq = (-rng.exponential(0.6, size=(B, K, g))).astype(np.float32)
        logq[0, 0, :] = logq[0, 1, :]                       # an exact tie between branches
        print(f"[case] branch prune B={B} K={K} gamma={g} tau={tau} keep={keep}", flush=True)
        mask, plen, conf = sv.specverify_branch_prune(to_dev(logq), float(np.log(tau)), keep)
        m_ref, l_ref, c_ref = bp.keep_branches(logq, float(np.log(tau)), keep)
        assert np.array_equal(conf.cpu().numpy(), c_ref)
        assert np.array_equal(plen.cpu().numpy(), l_ref)
        assert np.array_equal(mask.cpu().numpy().astype(bool), m_ref)


def test_non_finite_rows_set_the_row_error():
    # Reading of the input-error rule: a needed row whose largest logit is not finite (all
    # -inf, or any +inf or NaN entry) poisons its chains; a greedy row's draft rows are
    # never read, so a NaN there is no error.
    w = workloads.make("c3", B=7, V=9000, temps=("const", 0.7))
    w.temperature[2] = 0.0
    w.temperature[5] = 0.0
    nan, inf = (0x7FC0, 0x7F80) if w.dtype == "bf16" else (np.float32(np.nan), np.float32(np.inf))
    w.target[1, 2, 17] = nan               # one NaN among finite logits
    w.target[2, 1, 4000] = nan             # greedy row: NaN in the target row
    w.draft[3, 0, 1, 8191] = inf           # +inf in a draft row
    w.target[4, 0, :4096] = nan            # a whole chunk of NaN (its maximum reads -inf)
    w.draft[5, 0, 0, 5] = nan              # greedy batch row: draft logits are not needed
    w.target[6, 8, 100] = inf              # +inf in the bonus row
    print("[case] non-finite rows", flush=True)
    gpu = step_on_gpu(w)
    ref = _ref(w)
    assert ref["error"] == 4 and int(gpu["device_error"][0]) == 4
    assert np.array_equal(gpu["accept_len"], ref["accept_len"])
    for b in (1, 2, 3, 4, 6):
        assert gpu["accept_len"][b, 0] == -1 and gpu["out_token"][b, 0] == -1, b
    good = np.array([0, 5])
    compare_step({k: (v[good] if k not in ("device_error",) and v is not None else v)
                  for k, v in gpu.items()},
                 {k: (v[good] if isinstance(v, np.ndarray) and v.ndim >= 1 else v)
                  for k, v in ref.items()}, w.temperature[good])
    # the normalise entry point on the same rows: NaN where the oracle has no normaliser
    t = logits_to_dev(w.target, w.dtype)
    lnz, _ = sv.specverify_normalize(t, to_dev(w.temperature), want_argmax=True)
    torch.cuda.synchronize()
    rl, _ = oracle.normalize_rows(oracle.decode_logits(w.target, w.dtype), w.temperature[:, None])
    lnz = lnz.cpu().numpy()
    assert np.array_equal(np.isnan(lnz), np.isnan(rl))
    assert np.array_equal(np.isinf(lnz), np.isinf(rl))
    fin = np.isfinite(rl)
    assert np.all(np.abs(lnz[fin] - rl[fin]) <= LNZ_TOL)


def test_empty_residual_support_draws_from_p_unmasked():
    # Draft bytes equal to target bytes: ln q - ln p is exactly 0 for every id on both
    # sides, so the residual support is empty with no rounding ambiguity and the token is
    # the draw from p_n with the same noise. The oracle flags every such chain (an id
    # within eps of the support boundary), so this compares them unmasked; only chains
    # whose p_n draw has its runner-up within 2e-6 are left out, and they are counted.
    for V, dt in ((20000, "bf16"), (3001, "f32")):
        print(f"[case] empty support V={V} {dt}", flush=True)
        w = workloads.make("c3", B=16, V=V, gamma=4, dtype=dt, temps=("choice", (0.4, 1.0)))
        w.draft[:, 0] = w.target[:, :4]
        zt = oracle.decode_logits(w.target, w.dtype)
        zd = oracle.decode_logits(w.draft, w.dtype)
        T = w.temperature.astype(np.float64)
        lnz_t, am = oracle.normalize_rows(zt, T[:, None])
        lnz_d = lnz_t[:, None, :4].copy()
        n = np.random.default_rng(V).integers(0, 4, size=(w.B, 1))
        tok, _, empty = oracle.specverify.sample_tokens(zt, zd, T, lnz_t, lnz_d, am, n, w.seed,
                                                       w.pos0, np.arange(w.B)[:, None])
        assert empty.all()
        out = sv.specverify_residual_sample(
            logits_to_dev(w.target, w.dtype), logits_to_dev(w.draft, w.dtype), to_dev(w.temperature),
            to_dev(lnz_t), to_dev(lnz_d), to_dev(am.astype(np.int32)), to_dev(n.astype(np.int32)),
            w.seed, to_dev(w.pos0))
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        robust = np.ones(w.B, dtype=bool)
        for b in range(w.B):
            lp = zt[b, n[b, 0]] / T[b] - lnz_t[b, n[b, 0]]
            G = oracle.specverify.sampling_noise(w.seed, np.array([b]), w.pos0[b:b + 1] + n[b],
                                                 w.V)[0]
            sc = np.sort(lp + G)
            robust[b] = sc[-1] - sc[-2] >= 2e-6
        print(f"[parity] empty support: {int(robust.sum())} of {w.B} compared", flush=True)
        assert robust.sum() >= w.B - 1
        assert np.array_equal(got[robust, 0], tok[robust, 0]), (got.ravel(), tok.ravel())


def test_the_named_checked_build_is_the_one_loaded():
    """Under SPECVERIFY_LIBRARY=<libspecverify_checked.so> every GPU test ends with a
    zero count of failed device-side index checks (tests/conftest.py); this confirms
    that the counting build is the one in use."""
    import os

    named = os.environ.get("SPECVERIFY_LIBRARY")
    if not named:
        pytest.skip("the product build is loaded (SPECVERIFY_LIBRARY unset)")
    assert os.path.samefile(sv.LIBRARY, named)
    assert sv.check_count() is not None, "the named library has no device-side index checks"
