"""Helpers shared by the GPU parity tests: move a workload to the device, run the
HIP step, and compare it element by element with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import device_draft_verification_specverify_amd as sv

LNZ_TOL = 1e-5      # |d ln Z| <= 1e-5  <=>  Z within 1e-5 relative
LOGPROB_TOL = 1e-4  # gathered ln p / ln q, absolute


def device():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dev=None) -> torch.Tensor:
    dev = dev or device()
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def logits_to_dev(raw: np.ndarray, dtype: str, dev=None) -> torch.Tensor:
    if dtype == "bf16":
        return to_dev(raw.view(np.int16), dev).view(torch.bfloat16)
    return to_dev(raw.astype(np.float32), dev)


def step_on_gpu(w, target=None, draft=None, **kw):
    dev = device()
    t = logits_to_dev(w.target, w.dtype) if target is None else target
    d = logits_to_dev(w.draft, w.dtype) if draft is None else draft
    out = sv.specverify_step(t, d, to_dev(w.tokens), to_dev(w.temperature), w.seed,
                             to_dev(w.pos0), **kw)
    torch.cuda.synchronize(dev)
    res = {k: (None if v is None else v.cpu().numpy()) for k, v in vars(out).items()}
    return res


def flag_bound(chains: int) -> int:
    """Flagged chains a comparison may leave out: decisions within 1e-6 of a threshold are
    rare (about 1e-6 of probability mass per decision), so a handful at most."""
    return max(2, int(np.ceil(0.01 * chains)))


def compare_step(gpu: dict, ref: dict, temperature: np.ndarray, rows=None) -> dict:
    """Assert the spec bar; `rows` selects the batch rows the oracle computed. The
    flagged chains (left out of the exact comparison) are counted and bounded."""
    sel = slice(None) if rows is None else np.asarray(rows)
    g = {k: (v[sel] if isinstance(v, np.ndarray) and v.ndim >= 1 and k != "device_error" else v)
         for k, v in gpu.items()}
    T = np.asarray(temperature)[sel]
    sampled = T > 0
    ok = ~ref["flagged"]
    bad_n = np.argwhere((g["accept_len"] != ref["accept_len"]) & ok)
    bad_y = np.argwhere((g["out_token"] != ref["out_token"]) & ok)
    assert bad_n.size == 0, f"accept_len mismatches at {bad_n[:8].tolist()}"
    assert bad_y.size == 0, f"out_token mismatches at {bad_y[:8].tolist()}: gpu " \
        f"{g['out_token'][tuple(bad_y[0])]} oracle {ref['out_token'][tuple(bad_y[0])]}"
    stats = {"chains": int(ok.size), "flagged": int((~ok).sum())}
    assert stats["flagged"] <= flag_bound(stats["chains"]), stats
    if g.get("lnZ_target") is not None:
        dz = np.abs(g["lnZ_target"] - ref["lnZ_target"])
        assert np.all(dz[sampled] <= LNZ_TOL), f"max |d lnZ_t| = {dz[sampled].max()}"
        assert np.array_equal(g["lnZ_target"][~sampled], ref["lnZ_target"][~sampled])
        stats["max_dlnz_t"] = float(dz[sampled].max()) if sampled.any() else 0.0
    if g.get("lnZ_draft") is not None and sampled.any():
        dz = np.abs(g["lnZ_draft"][sampled] - ref["lnZ_draft"][sampled])
        assert np.all(dz <= LNZ_TOL), f"max |d lnZ_d| = {dz.max()}"
        stats["max_dlnz_d"] = float(dz.max())
    if g.get("logp") is not None:
        for key in ("logp", "logq"):
            a, b = g[key], ref[key]
            fin = np.isfinite(b)
            assert np.array_equal(np.isfinite(a), fin), key
            assert np.array_equal(a[~fin], b[~fin]), key
            d = np.abs(a[fin].astype(np.float64) - b[fin])
            assert d.size == 0 or d.max() <= LOGPROB_TOL, f"max |d {key}| = {d.max()}"
            stats[f"max_d{key}"] = float(d.max()) if d.size else 0.0
    return stats
