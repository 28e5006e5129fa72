"""specverify_step_noalloc -- the step for callers that cannot allocate -- against
specverify_step with a workspace, through the C ABI.

Two calls in a row on one GPU, the second with smaller inputs, so the second
runs on the scratch the first left behind; every output must be bit-identical
to the workspace step's (the same kernels in the same order) and within the
oracle's bar. Sizes beyond the scratch are refused before anything is enqueued.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import device_draft_verification_specverify_amd as sv
import oracle
import workloads
from gpu_helpers import compare_step, logits_to_dev, to_dev

pytestmark = pytest.mark.gpu


def _plans(w):
    args = (logits_to_dev(w.target, w.dtype), logits_to_dev(w.draft, w.dtype), to_dev(w.tokens),
            to_dev(w.temperature), w.seed, to_dev(w.pos0))
    return sv.StepPlan(*args), sv.StepPlan(*args, noalloc=True)


def test_noalloc_step_matches_the_workspace_step_on_consecutive_calls():
    cases = [workloads.make("c3", B=40, V=60000, temps=("choice", (0.0, 0.4, 1.0))),
             workloads.make("c2", B=5, V=3001, dtype="f32")]
    for i, w in enumerate(cases):
        print(f"[case] noalloc call {i}: B={w.B} K={w.K} gamma={w.gamma} V={w.V} {w.dtype}",
              flush=True)
        with_ws, no_ws = _plans(w)
        a = with_ws()
        b = no_ws()
        torch.cuda.synchronize()
        assert no_ws.ws is None
        for k, v in vars(a).items():
            if v is not None:
                assert torch.equal(v.nan_to_num(nan=-7.0), vars(b)[k].nan_to_num(nan=-7.0)), (i, k)
        got = {k: (None if v is None else v.cpu().numpy()) for k, v in vars(b).items()}
        ref = oracle.verify(w.target, w.draft, w.tokens, w.temperature, w.seed, w.pos0,
                            dtype=w.dtype)
        print(f"[parity] noalloc call {i}: {compare_step(got, ref, w.temperature)}", flush=True)
        assert int(got["device_error"][0]) == 0


def test_noalloc_step_refuses_sizes_beyond_its_scratch():
    B, K, g, V = 2048, 4, 8, 128256
    need = sv.workspace_size(B, K, g, V, sv.SV_BF16)
    assert need > sv.NOALLOC_SCRATCH_BYTES
    dev = torch.device("cuda:0")
    # stride-0 views: the refusal happens on the host before any device work
    t = torch.zeros((1, 1, V), dtype=torch.bfloat16, device=dev).expand(B, g + 1, V)
    d = torch.zeros((1, 1, 1, V), dtype=torch.bfloat16, device=dev).expand(B, K, g, V)
    toks = torch.zeros((B, K, g), dtype=torch.int32, device=dev)
    temp = torch.ones(B, dtype=torch.float32, device=dev)
    with pytest.raises(sv.SpecVerifyError, match="status -6"):
        sv.StepPlan(t, d, toks, temp, 1, None, noalloc=True)()
