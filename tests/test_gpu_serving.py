"""GPU: the usage patterns of a serving loop, through the C ABI.

* one workspace buffer shared by every entry point, in any order, stays valid
  (the per-chain counters sit at a fixed place and each call's first launch
  zeroes the ones it counts on; the acceptance sweep writes after them);
* two batches in flight on two streams, each with its own workspace, give the
  same outputs as one at a time;
* a step captured in a HIP graph replays with the eager step's outputs, replay
  after replay, with other eager work between the replays;
* the measurement hook marks the next streaming kernel's start and end, once.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import device_draft_verification_specverify_amd as sv
import workloads
from gpu_helpers import device, logits_to_dev, to_dev

pytestmark = pytest.mark.gpu


def _inputs(w):
    return (logits_to_dev(w.target, w.dtype), logits_to_dev(w.draft, w.dtype), to_dev(w.tokens),
            to_dev(w.temperature), to_dev(w.pos0))


def _host(out):
    return {k: (None if v is None else v.cpu().numpy()) for k, v in vars(out).items()}


def _same(a, b):
    for k in a:
        if a[k] is None:
            continue
        assert np.array_equal(a[k], b[k], equal_nan=True), k


def test_one_workspace_serves_every_entry_point():
    print("[case] shared workspace: step, accept_prob, step, normalize, steps", flush=True)
    w = workloads.make("c3", B=12)
    w2 = workloads.make("c2", B=9)
    dev = device()
    t, d, tok, temp, pos0 = _inputs(w)
    t2, d2, tok2, temp2, pos02 = _inputs(w2)
    need = max(sv.workspace_size(w.B, w.K, w.gamma, w.V, sv.SV_BF16),
               sv.workspace_size(w2.B, w2.K, w2.gamma, w2.V, sv.SV_BF16),
               sv.workspace_size(w.B, 0, 2 * w.gamma, w.V, sv.SV_BF16),
               int(sv.load_library().specverify_accept_prob_workspace_size(w.B, w.K, w.gamma,
                                                                             w.V, sv.SV_BF16)))
    # any contents: each call's first launch clears the counters it counts on
    shared = torch.full((need,), 0xFF, dtype=torch.uint8, device=dev)
    ref1 = _host(sv.StepPlan(t, d, tok, temp, w.seed, pos0)())
    ref2 = _host(sv.StepPlan(t2, d2, tok2, temp2, w2.seed, pos02)())
    p1 = sv.StepPlan(t, d, tok, temp, w.seed, pos0, ws=shared)
    p2 = sv.StepPlan(t2, d2, tok2, temp2, w2.seed, pos02, ws=shared)
    for _ in range(2):
        o1 = p1()
        sv.specverify_accept_prob(t, d, temp, o1.lnZ_target, torch.nan_to_num(o1.lnZ_draft),
                                  ws=shared)
        o2 = p2()
        stacked = torch.cat([t, d[:, 0]], dim=1).contiguous()
        sv.specverify_normalize(stacked, temp, ws=shared)
        _same(_host(p1()), ref1)
        _same(_host(p2()), ref2)
    torch.cuda.synchronize(dev)


def test_two_batches_on_two_streams():
    print("[case] two batches alternating on two streams", flush=True)
    dev = device()
    wa, wb = workloads.make("c3", B=16), workloads.make("c4", B=24)
    pa = sv.StepPlan(*_inputs(wa)[:4], wa.seed, _inputs(wa)[4])
    pb = sv.StepPlan(*_inputs(wb)[:4], wb.seed, _inputs(wb)[4])
    ref_a, ref_b = _host(pa()), _host(pb())
    s1, s2 = torch.cuda.Stream(dev), torch.cuda.Stream(dev)
    torch.cuda.synchronize(dev)
    for _ in range(10):
        pa(s1.cuda_stream)
        pb(s2.cuda_stream)
    torch.cuda.synchronize(dev)
    _same(_host(pa.out), ref_a)
    _same(_host(pb.out), ref_b)


def test_step_replays_from_a_graph():
    print("[case] step captured in a HIP graph, replayed", flush=True)
    dev = device()
    w = workloads.make("c3", B=8)
    t, d, tok, temp, pos0 = _inputs(w)
    plan = sv.StepPlan(t, d, tok, temp, w.seed, pos0)
    ref = _host(plan())
    s = torch.cuda.Stream(dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        plan(s.cuda_stream)              # warm-up on the capture stream
        torch.cuda.synchronize(dev)
        with torch.cuda.graph(g, stream=s):
            plan(s.cuda_stream)
    torch.cuda.synchronize(dev)
    for i in range(4):
        for v in vars(plan.out).values():
            if v is not None and v.dtype != torch.int32:
                v.fill_(float("nan"))
        plan.out.accept_len.fill_(-7)
        plan.out.out_token.fill_(-7)
        if plan.out.device_error is not None:
            plan.out.device_error.zero_()
        torch.cuda.synchronize(dev)
        g.replay()
        torch.cuda.synchronize(dev)
        _same(_host(plan.out), ref)
        # eager work between replays
        sv.StepPlan(t, d, tok, temp, w.seed + i, pos0)()


def test_timing_hook_marks_the_next_stream_kernel_once():
    print("[case] timing hook", flush=True)
    w = workloads.make("c3", B=16)
    t, d, tok, temp, pos0 = _inputs(w)
    plan = sv.StepPlan(t, d, tok, temp, w.seed, pos0)
    st = torch.cuda.current_stream(device())
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev[:2]:
        e.record(st)                      # the events exist once recorded
    plan()
    torch.cuda.synchronize()
    ev[2].record(st)
    sv.time_next_stream_kernel(ev[0], ev[1])
    plan()
    ev[3].record(st)
    torch.cuda.synchronize()
    kern, step = ev[0].elapsed_time(ev[1]), ev[2].elapsed_time(ev[3])
    assert 0.0 < kern < step, (kern, step)
    # one-shot: the next call leaves the two events where they were
    plan()
    torch.cuda.synchronize()
    assert ev[0].elapsed_time(ev[1]) == kern
