"""Seeded synthetic verification workloads.

Recipe (one independent random stream per (seed, purpose, index), drawn with
numpy's Philox bit generator, so a row can be regenerated on its own and rows
can be drawn by parallel threads):

* Gaussian logits: target ~ N(0, sigma_t^2) i.i.d.; draft = target + N(0, sigma_d^2).
* Zipf logits: target[v] = -1.1 * ln(rank[v]) + N(0, 0.3^2), with rank a random
  permutation of 1..V per row; draft = target + N(0, sigma_d^2).
* Values are drawn in float64, rounded to float32 (round-to-nearest-even), and
  for bf16 workloads rounded again to bf16 (round-to-nearest-even).
* The draft logits of branch k at position j are perturbed copies of the target
  row j of the same batch row (branches of one batch row share the target rows).
* Draft tokens are what a draft model sampling at the row's temperature would
  emit: an inverse-CDF draw from the softmax of the stored draft row at
  temperature T, or the stored draft row's argmax when T = 0.

Nothing here verifies anything: no normaliser, accept test or residual is
computed on the target side.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

GEN_TARGET = 16
GEN_DRAFT_NOISE = 17
GEN_PERM = 18
GEN_TEMP = 19
GEN_DRAFT_TOKEN = 20
GEN_POS = 21

VERIFY_SEED = 0xA5A51234_56789ABC

ZIPF_EXPONENT = 1.1
ZIPF_NOISE = 0.3

# The five workloads: vocabularies of the page models' families (32000, 128256,
# 151936), draft lengths 4-8, one to four draft branches per batch row.
CONFIGS = {
    "c1": dict(B=1, K=1, gamma=4, V=32000, dtype="f32", logits="gauss",
               sigma_t=2.0, sigma_d=0.5, temps=("const", 1.0)),
    "c2": dict(B=16, K=1, gamma=5, V=32000, dtype="bf16", logits="gauss",
               sigma_t=2.0, sigma_d=0.7, temps=("const", 0.7)),
    "c3": dict(B=64, K=1, gamma=8, V=128256, dtype="bf16", logits="zipf",
               sigma_d=1.0, temps=("choice", (0.1, 0.4, 0.7, 1.0))),
    "c4": dict(B=256, K=1, gamma=4, V=151936, dtype="bf16", logits="zipf",
               sigma_d=1.0, temps=("odd_greedy", 0.8)),
    "c5": dict(B=512, K=4, gamma=8, V=128256, dtype="bf16", logits="zipf",
               sigma_d=1.0, temps=("const", 0.7)),
}


@dataclass
class Workload:
    name: str
    B: int
    K: int
    gamma: int
    V: int
    dtype: str              # "f32" or "bf16"
    target: np.ndarray      # [B, gamma+1, V] float32, or uint16 bf16 bit patterns
    draft: np.ndarray       # [B, K, gamma, V] same storage as target
    tokens: np.ndarray      # [B, K, gamma] int32
    temperature: np.ndarray  # [B] float32 (0 = greedy row)
    pos0: np.ndarray        # [B] int64, sequence position of draft token 0
    seed: int               # 64-bit key of the verification's random stream

    @property
    def bytes_per_logit(self) -> int:
        return 4 if self.dtype == "f32" else 2


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _stream(seed: int, purpose: int, index: int) -> np.random.Generator:
    key = (int(seed) & 0xFFFFFFFFFFFFFFFF) | (((purpose << 48) | int(index)) << 64)
    return np.random.Generator(np.random.Philox(key=key))


def _temperature(cfg: dict, seed: int, b: int) -> float:
    kind, arg = cfg["temps"]
    if kind == "const":
        return float(arg)
    if kind == "choice":
        return float(arg[int(_stream(seed, GEN_TEMP, b).integers(0, len(arg)))])
    if kind == "odd_greedy":
        return 0.0 if b % 2 == 1 else float(arg)
    raise ValueError(kind)


def _store(raw64: np.ndarray, dtype: str) -> np.ndarray:
    f32 = raw64.astype(np.float32)
    return f32 if dtype == "f32" else round_to_bf16_bits(f32)


def _stored_as_f64(stored: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return stored.astype(np.float64)
    return bf16_bits_to_f32(stored).astype(np.float64)


def _draw_token(z: np.ndarray, T: float, rng: np.random.Generator) -> int:
    if T == 0.0:
        return int(np.argmax(z))
    w = np.exp((z - z.max()) / T)
    c = np.cumsum(w)
    x = int(np.searchsorted(c, rng.random() * c[-1], side="right"))
    return min(x, z.shape[0] - 1)


def make(name: str, B: int | None = None, V: int | None = None, gamma: int | None = None,
         K: int | None = None, seed: int = 0, threads: int | None = None,
         temps=None, dtype: str | None = None) -> Workload:
    """Draw workload `name` (c1..c5); keyword overrides give reduced or edge shapes."""
    cfg = dict(CONFIGS[name])
    for key, val in (("B", B), ("V", V), ("gamma", gamma), ("K", K), ("dtype", dtype), ("temps", temps)):
        if val is not None:
            cfg[key] = val
    B, K, g, Vv, dt = cfg["B"], cfg["K"], cfg["gamma"], cfg["V"], cfg["dtype"]
    store_dtype = np.float32 if dt == "f32" else np.uint16
    target = np.empty((B, g + 1, Vv), dtype=store_dtype)
    draft = np.empty((B, K, g, Vv), dtype=store_dtype)
    tokens = np.empty((B, K, g), dtype=np.int32)
    temperature = np.array([_temperature(cfg, seed, b) for b in range(B)], dtype=np.float32)
    pos0 = np.array([int(_stream(seed, GEN_POS, b).integers(0, 1 << 20)) for b in range(B)],
                    dtype=np.int64)
    zipf_base = None
    if cfg["logits"] == "zipf":
        zipf_base = -ZIPF_EXPONENT * np.log(np.arange(1, Vv + 1, dtype=np.float64))

    def target_row(b: int, j: int) -> np.ndarray:
        idx = b * (g + 1) + j
        noise = _stream(seed, GEN_TARGET, idx).standard_normal(Vv)
        if zipf_base is None:
            return cfg["sigma_t"] * noise
        perm = _stream(seed, GEN_PERM, idx).permutation(Vv)
        return zipf_base[perm] + ZIPF_NOISE * noise

    def fill(b: int) -> None:
        T = float(temperature[b])
        rows = [target_row(b, j) for j in range(g + 1)]
        for j in range(g + 1):
            target[b, j] = _store(rows[j], dt)
        for k in range(K):
            for j in range(g):
                idx = (b * K + k) * g + j
                raw = rows[j] + cfg["sigma_d"] * _stream(seed, GEN_DRAFT_NOISE, idx).standard_normal(Vv)
                draft[b, k, j] = _store(raw, dt)
                tokens[b, k, j] = _draw_token(_stored_as_f64(draft[b, k, j], dt), T,
                                              _stream(seed, GEN_DRAFT_TOKEN, idx))

    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    if threads <= 1 or B == 1:
        for b in range(B):
            fill(b)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(fill, range(B)))
    return Workload(name=name, B=B, K=K, gamma=g, V=Vv, dtype=dt, target=target, draft=draft,
                    tokens=tokens, temperature=temperature, pos0=pos0,
                    seed=VERIFY_SEED ^ (int(seed) & 0xFFFFFFFFFFFFFFFF))
