"""The seeded input generator: determinism, shapes, rounding and the per-config recipe."""
import numpy as np
import torch

import workloads
from workloads import synth


def test_deterministic_and_row_independent():
    a = workloads.make("c3", B=6, V=5000)
    b = workloads.make("c3", B=6, V=5000, threads=1)
    for f in ("target", "draft", "tokens", "temperature", "pos0"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    c = workloads.make("c3", B=3, V=5000)
    assert np.array_equal(c.target, a.target[:3]) and np.array_equal(c.draft, a.draft[:3])
    d = workloads.make("c3", B=6, V=5000, seed=1)
    assert not np.array_equal(d.target, a.target) and d.seed != a.seed


def test_shapes_and_dtypes_of_all_configs_reduced():
    for name, cfg in synth.CONFIGS.items():
        w = workloads.make(name, B=min(cfg["B"], 4), V=1024)
        B, K, g = w.B, w.K, w.gamma
        assert w.target.shape == (B, g + 1, 1024) and w.draft.shape == (B, K, g, 1024)
        assert w.target.dtype == (np.float32 if cfg["dtype"] == "f32" else np.uint16)
        assert w.tokens.shape == (B, K, g) and w.tokens.dtype == np.int32
        assert np.all((w.tokens >= 0) & (w.tokens < 1024))
        assert w.temperature.dtype == np.float32 and w.pos0.dtype == np.int64


def test_bf16_rounding_is_round_to_nearest_even():
    rng = np.random.default_rng(1)
    x = rng.normal(0, 10, size=200_000).astype(np.float32)
    ours = synth.round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(synth.bf16_bits_to_f32(ours),
                          torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_temperature_recipes():
    w3 = workloads.make("c3", V=256)
    assert set(np.unique(w3.temperature)) <= {np.float32(t) for t in (0.1, 0.4, 0.7, 1.0)}
    assert len(np.unique(w3.temperature)) == 4
    w4 = workloads.make("c4", B=10, V=256)
    assert np.all(w4.temperature[1::2] == 0) and np.all(w4.temperature[0::2] == np.float32(0.8))
    assert np.all(workloads.make("c5", B=3, V=256).temperature == np.float32(0.7))


def test_greedy_draft_tokens_are_draft_argmax_and_branches_share_target():
    w = workloads.make("c4", B=6, V=2000)
    z = synth.bf16_bits_to_f32(w.draft)
    for b in range(1, 6, 2):
        assert np.array_equal(w.tokens[b, 0], np.argmax(z[b, 0], axis=-1))
    w5 = workloads.make("c5", B=2, V=2000)
    zt = synth.bf16_bits_to_f32(w5.target).astype(np.float64)
    zd = synth.bf16_bits_to_f32(w5.draft).astype(np.float64)
    diff = zd - zt[:, None, :-1]
    assert abs(diff.std() - 1.0) < 0.02             # draft = target + N(0, 1)
    assert not np.array_equal(w5.draft[:, 0], w5.draft[:, 1])


def test_zipf_rows_are_permuted_ranks():
    w = workloads.make("c3", B=1, V=4096)
    z = synth.bf16_bits_to_f32(w.target[0, 0]).astype(np.float64)
    srt = np.sort(z)[::-1]
    base = -1.1 * np.log(np.arange(1, 4097))
    assert np.corrcoef(srt, base)[0, 1] > 0.99
    assert np.argmax(z) != 0 or np.argmax(synth.bf16_bits_to_f32(w.target[0, 1])) != 0
