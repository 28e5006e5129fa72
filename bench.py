"""Benchmark: one batched speculative-sampling verification step per timed step.

Workload: B=64 rows, gamma=8 draft tokens, V=128256, bf16 Zipf-shaped logits
(ranks permuted per row, per-row temperature in {0.1, 0.4, 0.7, 1.0}); draft =
target + N(0, 1). Synthetic, seeded, generated on the host then copied to HBM
before timing.

Prints one JSON line: verified draft tokens/s (B*gamma per step) and the HBM
roofline of the dominant kernel, plus the fp64 CPU oracle timed on a bounded
sample as a reported baseline, and `parity`: per workload, the chains whose
accept length or token differ from the oracle's, and the chains left out
because a decision lies within 1e-6 of its threshold. `per_config` adds every workload (C1-C5, and the
accept test alone on C4's log-probabilities) timed cold: before each of the
timed reps a 512 MiB buffer is rewritten, which evicts the 256 MB last-level
cache and the L2s, and HIP events bracket the step alone (median, p10, p90).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--copies C] [--no-cpu]
                    [--per-config all|none|c1,c3,...] [--reps R]
"""
from __future__ import annotations

import argparse
import concurrent.futures
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import device_draft_verification_specverify_amd as sv  # noqa: E402
import workloads  # noqa: E402

METRIC = "verified draft tokens/s + HBM GB/s (% of peak) at B=64, γ=8, V=128256 bf16"
HBM_PEAK_GBPS = 8000.0
COPY_BYTES = 1 << 28


def algorithmic_bytes(w) -> int:
    """Every logit the rule needs, read once, plus tokens, temperatures and outputs."""
    e = w.bytes_per_logit
    sampled = int((w.temperature > 0).sum())
    logits = w.B * (w.gamma + 1) * w.V * e + sampled * w.K * w.gamma * w.V * e
    scalars = w.B * w.K * w.gamma * 4 + w.B * 4 + w.B * 8 + 2 * w.B * w.K * 4
    return logits + scalars


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "stream_kernel_B64_rows17_V128256_bf16_traffic.md")
KERNEL_SOURCE = os.path.join(ROOT, "device_draft_verification_specverify_amd", "csrc",
                             "specverify.hip")


def measured_traffic():
    """HBM bytes per launch of the streaming kernel from the committed counter runs
    (FETCH_SIZE + WRITE_SIZE, scaled by a copy of known size), or None when they
    were taken on another version of the kernel source."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            fields = dict(re.findall(r"^- (\w+): (\S+)\s*$", f.read(), re.M))
        with open(KERNEL_SOURCE, "rb") as f:
            digest = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    if fields.get("source_sha256") != digest or "traffic_bytes_per_launch" not in fields:
        return None
    return float(fields["traffic_bytes_per_launch"])


def stacked_inputs(w, dev):
    """Target and draft rows of one copy in a single [B, 2*gamma+1, V] buffer; returns views."""
    raw = np.concatenate([w.target, w.draft[:, 0]], axis=1)
    buf = torch.from_numpy(raw.view(np.int16)).to(dev).view(torch.bfloat16)
    g = w.gamma
    return buf, buf[:, : g + 1], buf[:, g + 1:].unsqueeze(1)


def _oracle_rows(w, rows):
    import oracle

    return oracle.verify(w.target[rows], w.draft[rows], w.tokens[rows], w.temperature[rows],
                         w.seed, w.pos0[rows], batch_index=rows, dtype=w.dtype)


def cpu_baseline(w, min_seconds: float = 10.0, max_reps: int = 300):
    """The oracle as it is, on the host's cores: one thread per slice of batch rows
    (NumPy releases the GIL inside its array operations), whole steps repeated
    until min_seconds have passed. Returns the figure and the last step's oracle
    accept lengths, tokens and flags."""
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    slices = [r for r in np.array_split(np.arange(w.B), threads) if len(r)]

    reps, t0 = 0, time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(slices)) as ex:
        while reps < max_reps:
            outs = list(ex.map(lambda r: _oracle_rows(w, r), slices))
            reps += 1
            if time.perf_counter() - t0 >= min_seconds:
                break
    dt = (time.perf_counter() - t0) / reps
    ref = {k: np.concatenate([o[k] for o in outs]) for k in ("accept_len", "out_token", "flagged")}
    return {"value": w.B * w.K * w.gamma / dt, "unit": "tokens/s", "cores": len(slices),
            "kind": "oracle",
            "sample": f"{reps} full step(s) of the benchmark workload ({w.B} chains, "
                      f"{w.B * w.K * w.gamma} draft tokens), NumPy float64, one thread per "
                      f"slice of batch rows",
            "seconds_per_step": dt, "gbps": algorithmic_bytes(w) / dt / 1e9}, ref


# Batch rows of each workload whose chains the parity count covers (all of the small
# ones; a seeded sample of the large ones, so the oracle finishes in seconds).
PARITY_ROWS = {"c4": 32, "c5": 16}


def parity_rows(w) -> np.ndarray:
    n = PARITY_ROWS.get(w.name)
    if n is None or n >= w.B:
        return np.arange(w.B)
    return np.sort(np.random.default_rng(1234).choice(w.B, n, replace=False))


def parity_sample(w, out) -> dict:
    """What the oracle needs to check a GPU step on parity_rows(w): the rows' inputs and
    the GPU's accept lengths and tokens for them."""
    rows = parity_rows(w)
    return {"rows": rows, "B": w.B, "name": w.name, "seed": w.seed, "dtype": w.dtype,
            "target": w.target[rows], "draft": w.draft[rows], "tokens": w.tokens[rows],
            "temperature": w.temperature[rows], "pos0": w.pos0[rows],
            "accept_len": out.accept_len.cpu().numpy()[rows],
            "out_token": out.out_token.cpu().numpy()[rows]}


def parity_count(gpu_n, gpu_y, ref, rows_note: str) -> dict:
    """Mismatches of the GPU step against the oracle on chains whose decisions are not
    within 1e-6 of a threshold, and the number of such excluded (flagged) chains."""
    ok = ~ref["flagged"]
    return {"chains": int(ok.size), "rows": rows_note,
            "accept_len_mismatches": int(((gpu_n != ref["accept_len"]) & ok).sum()),
            "out_token_mismatches": int(((gpu_y != ref["out_token"]) & ok).sum()),
            "flagged_excluded": int(ref["flagged"].sum())}


def parity_of_samples(samples: dict) -> dict:
    import oracle

    res = {}
    for name, smp in samples.items():
        rows = smp["rows"]
        ref = oracle.verify(smp["target"], smp["draft"], smp["tokens"], smp["temperature"],
                            smp["seed"], smp["pos0"], batch_index=rows, dtype=smp["dtype"])
        note = "all" if rows.size == smp["B"] else f"{rows.size} of {smp['B']} (seeded sample)"
        res[name] = parity_count(smp["accept_len"], smp["out_token"], ref, note)
    return res


def progress(msg: str) -> None:
    """One line on stderr as each phase ends (the JSON line alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def device_logits(raw: np.ndarray, dtype: str, dev) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(raw.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(raw).to(dev)


def pct(xs, q) -> float:
    return float(np.percentile(np.asarray(xs), q))


def cold_times_us(fn, reps: int, warmup: int, scratch: torch.Tensor, stream) -> list:
    """HIP-event time of fn() per rep, each after a 512 MiB rewrite of scratch."""
    for _ in range(warmup):
        fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for i in range(reps):
        scratch.fill_(i & 0xFF)
        ev[i][0].record(stream)
        fn()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return [1e3 * a.elapsed_time(b) for a, b in ev]


def per_config(names, reps: int, warmup: int, dev, samples: dict | None = None) -> dict:
    """Every workload's step timed cold; C4 also times the accept test alone. With
    `samples`, each workload's parity_sample of its last timed step is kept there."""
    stream = torch.cuda.current_stream(dev)
    scratch = torch.empty(1 << 29, dtype=torch.uint8, device=dev)
    res = {}
    for name in names:
        w = workloads.make(name)
        tgt = device_logits(w.target, w.dtype, dev)
        dft = device_logits(w.draft, w.dtype, dev)
        tokens = torch.from_numpy(w.tokens).to(dev)
        temp = torch.from_numpy(w.temperature).to(dev)
        pos0 = torch.from_numpy(w.pos0).to(dev)
        plan = sv.StepPlan(tgt, dft, tokens, temp, w.seed, pos0)
        us = cold_times_us(plan, reps, warmup, scratch, stream)
        med = pct(us, 50)
        # back-to-back steps on the same inputs (warm caches), for the launch-bound sizes
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(20):
            plan()
        e1.record(stream)
        torch.cuda.synchronize()
        warm = 1e3 * e0.elapsed_time(e1) / 20
        nbytes = algorithmic_bytes(w)
        entry = {"B": w.B, "K": w.K, "gamma": w.gamma, "V": w.V, "logits": w.dtype,
                 "us_median": med, "us_p10": pct(us, 10), "us_p90": pct(us, 90),
                 "us_warm_back_to_back": warm,
                 "tokens_per_s": w.B * w.K * w.gamma / (med * 1e-6),
                 "bytes_min": nbytes, "hbm_gbps": nbytes / (med * 1e-6) / 1e9,
                 "hbm_frac_of_peak": nbytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                 "device_error": int(plan.out.device_error.item())}
        if samples is not None:
            samples[name] = parity_sample(w, plan.out)
        progress(f"{name}: step {med:.1f} us cold")
        # the acceptance probability and accept-length law of the same step's rows
        lz_t = plan.out.lnZ_target.clone()
        lz_d = torch.nan_to_num(plan.out.lnZ_draft, nan=0.0)
        aws = sv.accept_prob_workspace(w.B, w.K, w.gamma, w.V, plan.dtype, dev)
        ap = cold_times_us(lambda: sv.specverify_accept_prob(tgt, dft, temp, lz_t, lz_d, ws=aws),
                           reps, warmup, scratch, stream)
        ap_bytes = (w.B * w.gamma * w.V + w.B * w.K * w.gamma * w.V) * w.bytes_per_logit
        entry["accept_prob"] = {"us_median": pct(ap, 50), "us_p10": pct(ap, 10),
                                "us_p90": pct(ap, 90), "bytes_min": ap_bytes,
                                "hbm_gbps": ap_bytes / (pct(ap, 50) * 1e-6) / 1e9}
        del aws
        # residual top-F candidates of every outcome (geometric fan-out, 8 per outcome on
        # average) and the cache lookup of this step's outcomes
        fan = sv.geometric_fanout(w.gamma, 8 * (w.gamma + 1), 0.6)
        tf = cold_times_us(lambda: sv.specverify_residual_topf(tgt, dft, temp, lz_t, lz_d, fan),
                           reps, warmup, scratch, stream)
        cand, _ = sv.specverify_residual_topf(tgt, dft, temp, lz_t, lz_d, fan)
        lk = cold_times_us(lambda: sv.specverify_cache_lookup(cand, fan, plan.out.accept_len,
                                                              plan.out.out_token),
                           reps, warmup, scratch, stream)
        tf_bytes = (w.B * (w.gamma + 1) * w.V + w.B * w.K * w.gamma * w.V) * w.bytes_per_logit
        entry["residual_topf"] = {"fanout": fan, "us_median": pct(tf, 50), "us_p10": pct(tf, 10),
                                  "us_p90": pct(tf, 90), "bytes_min": tf_bytes,
                                  "hbm_gbps": tf_bytes / (pct(tf, 50) * 1e-6) / 1e9}
        entry["cache_lookup"] = {"us_median": pct(lk, 50), "us_p10": pct(lk, 10),
                                 "us_p90": pct(lk, 90)}
        del cand
        res[name] = entry
        if name == "c4":
            # the accept test alone on this step's [B, K, gamma] log-probabilities
            lp, lq = plan.out.logp.clone(), plan.out.logq.clone()
            acc = cold_times_us(lambda: sv.specverify_accept(lp, lq, w.seed, pos0), reps, warmup,
                                scratch, stream)
            res["c4_accept_only"] = {"B": w.B, "K": w.K, "gamma": w.gamma,
                                     "us_median": pct(acc, 50), "us_p10": pct(acc, 10),
                                     "us_p90": pct(acc, 90),
                                     "decisions_per_call": w.B * w.K * w.gamma}
        del plan, tgt, dft
        torch.cuda.empty_cache()
    return res


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=1000,
                    help="untimed steps first; the clocks settle within a few hundred steps")
    ap.add_argument("--copies", type=int, default=4,
                    help="input copies cycled so consecutive steps never reuse cached logits")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--per-config", default="all",
                    help="'all', 'none', or a comma list of c1..c5 timed cold after the main run")
    ap.add_argument("--reps", type=int, default=50, help="timed reps per workload in per_config")
    ap.add_argument("--no-two-stream", action="store_true",
                    help="skip the two-batch, two-stream context figure (profiled runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help=f"after timing, copy {COPY_BYTES} bytes three times (counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the verification path runs on a single device "
              "(sharding is described, not built); use --gpus 1", file=sys.stderr)
        return 2

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workloads.make("c3")
    copies = []
    for c in range(args.copies):
        buf, tgt, dft = stacked_inputs(w, dev)
        copies.append((buf, tgt, dft))
    tokens = torch.from_numpy(w.tokens).to(dev)
    temp = torch.from_numpy(w.temperature).to(dev)
    pos0 = torch.from_numpy(w.pos0).to(dev)
    plans = [sv.StepPlan(t, d, tokens, temp, w.seed, pos0) for (_, t, d) in copies]
    stream = torch.cuda.current_stream(dev)

    for i in range(args.warmup):
        plans[i % len(plans)]()
    torch.cuda.synchronize(dev)

    # Timed region: exactly `steps` steps, bracketed by device synchronisation.
    t0 = time.perf_counter()
    for i in range(args.steps):
        plans[i % len(plans)]()
    torch.cuda.synchronize(dev)
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / args.steps
    progress(f"timed region: {args.steps} steps, {1e3 * ms_per_step:.1f} us per step")

    # Context only (not `value`): two independent batches alternating on two streams,
    # so that one batch's draws can overlap the other's streaming (as two micro-batches
    # of a server would); each plan has its own workspace.
    two_stream_ms = None
    if not args.no_two_stream:
        side = torch.cuda.Stream(dev)
        streams = [stream, side]
        for i in range(args.warmup):
            plans[i % len(plans)](streams[i % 2].cuda_stream)
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        for i in range(args.steps):
            plans[i % len(plans)](streams[i % 2].cuda_stream)
        torch.cuda.synchronize(dev)
        two_stream_ms = 1e3 * (time.perf_counter() - t0) / args.steps

    # Dominant kernel: the streaming normaliser inside the same steps, timed with HIP
    # events that the library records on its launch stream just before and after that
    # kernel (the same steps again, after the timed region, so the event records do
    # not touch `value`).
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for a, b in ev:  # the events exist once recorded
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize(dev)
    for i in range(args.steps):
        sv.time_next_stream_kernel(*ev[i])
        plans[i % len(plans)]()
    torch.cuda.synchronize(dev)
    kern_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    progress(f"stream kernel: {1e3 * kern_ms:.1f} us per launch")

    if args.copy_calibration:
        # A plain device copy of known size, for scaling the HBM byte counters.
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize(dev)

    out = plans[0].out
    err = int(out.device_error.item())
    bytes_min = algorithmic_bytes(w)
    # every target row and every sampled batch row's draft rows, read once
    kernel_bytes = (w.B * (w.gamma + 1) + int((w.temperature > 0).sum()) * w.K * w.gamma) \
        * w.V * w.bytes_per_logit
    achieved = kernel_bytes / (kern_ms * 1e-3) / 1e9
    tokens_per_step = w.B * w.K * w.gamma
    value = tokens_per_step / (ms_per_step * 1e-3)
    step_gbps = bytes_min / (ms_per_step * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "B=64, gamma=8, V=128256 bf16 Zipf logits, per-row T in "
                               "{0.1,0.4,0.7,1.0}, K=1", "B": w.B, "K": w.K, "gamma": w.gamma,
                   "V": w.V, "logits": "bf16", "input_copies_cycled": args.copies},
        "two_batch_streams": None if two_stream_ms is None else {
            "ms_per_step": two_stream_ms, "tokens_per_s": tokens_per_step / (two_stream_ms * 1e-3),
            "note": "context only: two independent batches alternating on two streams; value is "
                    "one step at a time"},
        "hbm_gbps": step_gbps,
        "hbm_frac_of_peak": step_gbps / HBM_PEAK_GBPS,
        "bytes_min_per_step": bytes_min,
        "accepted_tokens_per_step": int((out.accept_len.clamp(min=0) + 1).sum().item()),
        "device_error": err,
        "roofline": {"bound": "hbm", "kernel": "stream_kernel",
                     "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": measured_traffic(),
                     "bytes_per_launch": kernel_bytes, "avg_launch_ms": kern_ms,
                     "timing": "HIP events recorded by the library around the stream kernel "
                               f"inside {args.steps} steps"},
    }
    gpu_n = out.accept_len.cpu().numpy()
    gpu_y = out.out_token.cpu().numpy()
    samples = {} if not args.no_cpu else None
    if args.per_config != "none":
        names = (list(workloads.CONFIGS) if args.per_config == "all"
                 else [n for n in args.per_config.split(",") if n])
        line["per_config"] = per_config(names, args.reps, 10, dev, samples)
    if not args.no_cpu:
        # the oracle's leg: its timing, and the parity of the GPU steps above against it
        line["cpu_baseline"], ref = cpu_baseline(w)
        progress("oracle timed")
        parity = {"c3_timed_step": parity_count(gpu_n, gpu_y, ref, "all")}
        parity.update(parity_of_samples(samples))
        line["parity"] = parity
    else:
        line["parity"] = None
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
