"""Property-based parity sweep of the fused step (FlashSpec, technical summary,
section 3 "Correctness and testing": property-based tests over batch sizes and
speculation lengths with the Hypothesis library).

Derandomised (a fixed seed, so every run draws the same 30 cases) and without
shrinking, so a failure stops the sweep at once. Each case draws a batch size,
branch count, draft length, vocabulary (not always a multiple of 8), logit
type, dtype, a set of temperatures (greedy, very cold, hot) and whether all
batch rows share one target context (stride 0); the oracle checks up to six of
its batch rows, and every chain's outputs are checked for range.
"""
from __future__ import annotations

import numpy as np
import pytest
from hypothesis import HealthCheck, Phase, given, settings
from hypothesis import strategies as st

import oracle
import workloads
from gpu_helpers import compare_step, logits_to_dev, step_on_gpu

pytestmark = pytest.mark.gpu

TEMPS = (0.0, 1e-2, 0.1, 0.7, 1.0, 3.0)
LOGIT_BUDGET = 12_000_000          # logits per case, so a case draws and checks in seconds
ROW_BUDGET = 6_000                 # logit rows per case (the generator draws row by row)


@st.composite
def cases(draw):
    V = draw(st.one_of(st.integers(2, 64), st.integers(65, 8192), st.integers(8193, 160_000)))
    K = draw(st.integers(1, 4))
    gamma = draw(st.integers(1, 16))
    per_b = gamma + 1 + K * gamma
    bmax = max(1, min(600, LOGIT_BUDGET // (per_b * V), ROW_BUDGET // per_b))
    B = draw(st.integers(1, bmax))
    temps = tuple(sorted(draw(st.sets(st.sampled_from(TEMPS), min_size=1, max_size=3))))
    return dict(B=B, K=K, gamma=gamma, V=V, temps=temps,
                dtype=draw(st.sampled_from(("bf16", "f32"))),
                logits=draw(st.sampled_from(("c2", "c3"))),
                broadcast=draw(st.booleans()))


@settings(max_examples=30, derandomize=True, deadline=None, database=None,
          phases=[Phase.explicit, Phase.generate],
          suppress_health_check=list(HealthCheck))
@given(case=cases())
def test_step_matches_oracle_on_drawn_shapes(case):
    print(f"[case] hypothesis {case}", flush=True)
    w = workloads.make(case["logits"], B=case["B"], K=case["K"], gamma=case["gamma"],
                       V=case["V"], dtype=case["dtype"], temps=("choice", case["temps"]),
                       threads=8)
    target = None
    if case["broadcast"]:
        w.target[:] = w.target[0]                      # one shared context, read with stride 0
        target = logits_to_dev(w.target[:1], w.dtype).expand(w.B, w.gamma + 1, w.V)
    gpu = step_on_gpu(w, target=target)
    n, y = gpu["accept_len"], gpu["out_token"]
    assert int(gpu["device_error"][0]) == 0
    assert np.all((n >= 0) & (n <= w.gamma)) and np.all((y >= 0) & (y < w.V))
    rows = np.unique(np.concatenate([[0, w.B - 1],
                                     np.random.default_rng(w.B).integers(0, w.B, size=4)]))
    ref = oracle.verify(w.target[rows], w.draft[rows], w.tokens[rows], w.temperature[rows],
                        w.seed, w.pos0[rows], batch_index=rows, dtype=w.dtype)
    stats = compare_step(gpu, ref, w.temperature, rows)
    print(f"[parity] hypothesis: {stats}", flush=True)
