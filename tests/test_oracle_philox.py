"""Pins for the oracle's Philox4x32-10 stream, uniform map and Gumbel noise.

The oracle implements Philox4x32-10 from its published definition (Salmon et
al., SC'11). It is pinned here against an independent implementation, the
rocRAND library's Philox4x32-10 engine (compiled on the host from its header),
and by distribution tests of the uniform and Gumbel maps.
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
from scipy import stats

from oracle import philox

ROCRAND_PROGRAM = r"""
#include <rocrand/rocrand_kernel.h>
#include <cstdio>
#include <cstdint>
#include <vector>
// stdin: n, then n records of (c0, c1, c2, c3, k0, k1) as uint32; stdout: 4 words per record.
// rocRAND's engine keys (k0, k1) from the 64-bit seed, places the subsequence in counter
// words 2-3 and (skipped elements)/4 in counter words 0-1, and returns word (skip % 4) of the
// block. Counter word 1 is reached by skips of at most 2^62 elements (no 64-bit overflow).
int main() {
  uint64_t n;
  if (fread(&n, 8, 1, stdin) != 1) return 1;
  std::vector<uint32_t> in(6 * n), out(4 * n);
  if (fread(in.data(), 4, 6 * n, stdin) != 6 * n) return 2;
  for (uint64_t i = 0; i < n; ++i) {
    const uint32_t* r = &in[6 * i];
    unsigned long long seed = (unsigned long long)r[4] | ((unsigned long long)r[5] << 32);
    unsigned long long sub = (unsigned long long)r[2] | ((unsigned long long)r[3] << 32);
    rocrand_state_philox4x32_10 st;
    rocrand_init(seed, sub, 4ull * (unsigned long long)r[0], &st);
    skipahead((unsigned long long)(r[1] & 0x0FFFFFFFu) << 34, &st);
    for (uint32_t s = 0; s < (r[1] >> 28); ++s) skipahead(1ull << 62, &st);
    for (int w = 0; w < 4; ++w) out[4 * i + w] = rocrand(&st);
  }
  fwrite(out.data(), 4, 4 * n, stdout);
  return 0;
}
"""


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand) and os.path.exists("/opt/rocm/include/rocrand/rocrand_kernel.h"):
            return cand
    return None


@pytest.fixture(scope="module")
def rocrand_blocks():
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc / rocRAND headers not available")
    tmp = tempfile.mkdtemp(prefix="philox_pin_")
    src = os.path.join(tmp, "pin.cpp")
    exe = os.path.join(tmp, "pin")
    with open(src, "w") as f:
        f.write(ROCRAND_PROGRAM)
    subprocess.run([hipcc, "-O2", src, "-o", exe], check=True, capture_output=True)

    def run(words6: np.ndarray) -> np.ndarray:
        words6 = np.ascontiguousarray(words6, dtype=np.uint32)
        n = words6.shape[0]
        payload = np.uint64(n).tobytes() + words6.tobytes()
        res = subprocess.run([exe], input=payload, check=True, capture_output=True)
        return np.frombuffer(res.stdout, dtype=np.uint32).reshape(n, 4)
    yield run
    shutil.rmtree(tmp, ignore_errors=True)


def test_philox_matches_rocrand_on_random_and_edge_counters(rocrand_blocks):
    rng = np.random.default_rng(20260101)
    rand = rng.integers(0, 2 ** 32, size=(200_000, 6), dtype=np.uint64).astype(np.uint32)
    edge_vals = np.array([0, 1, 2, 3, 0x7FFFFFFF, 0x80000000, 0xFFFFFFFE, 0xFFFFFFFF], dtype=np.uint32)
    edges = np.array(np.meshgrid(*([edge_vals[[0, 1, 7]]] * 6), indexing="ij")).reshape(6, -1).T
    # the counter layout the verification uses: small c0, positions, chain rows, purposes
    layout = np.stack([
        np.arange(4096) % 40000, 937971 + np.arange(4096) % 9, np.arange(4096) // 9 % 2048,
        np.arange(4096) % 2, np.full(4096, 0x56789ABC), np.full(4096, 0xA5A51234)], axis=1)
    words6 = np.concatenate([rand, edges.astype(np.uint32), layout.astype(np.uint32)])
    ref = rocrand_blocks(words6)
    got = np.stack(philox.block(*[words6[:, i] for i in range(6)]), axis=1)
    mism = np.nonzero(np.any(got != ref, axis=1))[0]
    assert mism.size == 0, f"{mism.size} mismatching blocks, first at {words6[mism[0]]}"


def test_uniform_map_range_and_exactness():
    w = np.array([0, 1, 511, 512, 0x7FFFFFFF, 0x80000000, 0xFFFFFFFF], dtype=np.uint32)
    u = philox.uniform(w)
    assert u[0] == 2.0 ** -24 and u[1] == 2.0 ** -24 and u[2] == 2.0 ** -24
    assert u[3] == 3 * 2.0 ** -24
    assert u[-1] == 1.0 - 2.0 ** -24
    assert np.all((u > 0) & (u < 1))
    assert np.array_equal(u.astype(np.float32).astype(np.float64), u)   # exact in float32
    # 2^23 equally spaced values: the map is the midpoint of the top-23-bit cell
    assert np.allclose((u - 2.0 ** -24) * 2 ** 23, w >> 9)


def test_uniformity_chi2_over_the_verification_layout():
    # 2^20 blocks across chain rows and positions, all four words: 4M uniforms, 1024 bins
    r = np.arange(1024)[:, None]
    pos = np.arange(1024)[None, :] + 123456
    words = np.stack(philox.block(np.arange(1024)[None, :] % 7, pos, r, 1, 0x9E3779B9, 0x12345678))
    u = philox.uniform(words.ravel())
    counts = np.bincount(np.minimum((u * 1024).astype(np.int64), 1023), minlength=1024)
    pval = stats.chisquare(counts).pvalue
    assert pval > 1e-3, pval


def test_purposes_and_fields_decorrelated():
    base = dict(c0=np.arange(100_000), c1=7, c2=3, c3=0)
    a = philox.block(base["c0"], 7, 3, 0, 11, 13)[0].astype(np.float64)
    b = philox.block(base["c0"], 7, 3, 1, 11, 13)[0].astype(np.float64)   # other purpose
    c = philox.block(base["c0"], 8, 3, 0, 11, 13)[0].astype(np.float64)   # next position
    for x in (b, c):
        rho = np.corrcoef(a, x)[0, 1]
        assert abs(rho) < 0.02, rho
        assert np.mean(a == x) < 1e-3


def test_gumbel_noise_distribution_and_log_accuracy():
    words = np.stack(philox.block(np.arange(250_000), 5, 9, 1, 1, 2)).ravel()
    g = philox.gumbel(philox.uniform(words))
    assert stats.kstest(g, stats.gumbel_r.cdf).pvalue > 0.01
    # -ln u near 1: the log1p branch keeps full relative accuracy where u - 1 is exact
    u = 1.0 - np.array([2.0 ** -24, 3 * 2.0 ** -24, 2.0 ** -10, 0.25])
    e = philox.neg_log_uniform(u)
    t = 1.0 - u
    series = t + t ** 2 / 2 + t ** 3 / 3 + t ** 4 / 4 + t ** 5 / 5
    assert np.allclose(e[:3], series[:3], rtol=1e-15, atol=0)
    assert np.isclose(e[3], np.log(4.0 / 3.0), rtol=1e-15)
