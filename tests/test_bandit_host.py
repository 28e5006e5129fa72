"""The library's draft selector (host C ABI, no GPU) against the oracle's (CPU only).

The same reward sequence drives both; UCB1 and Thompson sampling must pick the
same arms at every step (same published algorithms, same Philox4x32-10 stream,
float64 throughout, no contraction on the library side).
"""
import ctypes

import numpy as np
import pytest

import device_draft_verification_specverify_amd as sv
from oracle import bandit as bd


@pytest.mark.parametrize("policy,arms,seed", [
    (sv.BANDIT_UCB1, 3, 0), (sv.BANDIT_UCB1, 7, 0), (sv.BANDIT_THOMPSON, 3, 11),
    (sv.BANDIT_THOMPSON, 5, 2 ** 63 + 5),
])
def test_selections_match_the_oracle(policy, arms, seed):
    rng = np.random.default_rng(seed & 0xFFFF)
    means = rng.uniform(0.2, 0.9, size=arms)
    lib_b = sv.Bandit(arms, policy, seed=seed)
    ora_b = bd.Bandit(arms, policy, seed=seed)
    for step in range(250):
        a1, a2 = lib_b.select(), ora_b.select()
        assert a1 == a2, (step, a1, a2)
        # fractional rewards, as accepted fractions are
        r = float(np.clip(means[a1] + rng.normal(0, 0.1), 0, 1))
        lib_b.update(a1, r)
        ora_b.update(a2, r)
    for i in range(arms):
        pulls, total = lib_b.stats(i)
        assert pulls == ora_b.pulls[i] and abs(total - ora_b.sums[i]) < 1e-12


def test_step_reward_matches_the_oracle():
    n = np.array([[3, 0], [8, 8], [-1, 5]], dtype=np.int32)
    assert sv.step_reward(n, 8) == bd.step_reward(n, 8)
    assert sv.step_reward([9, 2], 8) == (8 + 2) / 16


def test_bandit_validation():
    lib = sv.load_library()
    assert lib.specverify_bandit_state_size(0) == 0
    assert lib.specverify_bandit_state_size(257) == 0
    n = lib.specverify_bandit_state_size(4)
    buf = ctypes.create_string_buffer(n)
    assert lib.specverify_bandit_init(buf, n, 4, 9, 0, 2.0) == -1
    assert lib.specverify_bandit_init(buf, n, 4, 0, 0, 0.0) == -1
    assert lib.specverify_bandit_init(buf, n - 1, 4, 0, 0, 2.0) == -3
    assert lib.specverify_bandit_init(None, n, 4, 0, 0, 2.0) == -1
    arm = ctypes.c_int32()
    fresh = ctypes.create_string_buffer(n)
    assert lib.specverify_bandit_select(fresh, ctypes.byref(arm)) == -1   # not initialised
    assert lib.specverify_bandit_init(buf, n, 4, 0, 0, 2.0) == 0
    assert lib.specverify_bandit_update(buf, 4, 0.5) == -1
    assert lib.specverify_bandit_update(buf, 0, 1.5) == -1
    assert lib.specverify_bandit_update(buf, 0, float("nan")) == -1
    out = ctypes.c_double()
    assert lib.specverify_step_reward(None, 3, 4, ctypes.byref(out)) == -1
