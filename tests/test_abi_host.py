"""The C ABI on the host (no GPU needed): the library loads, exports every
symbol its header declares, sizes workspaces, and rejects bad arguments before
touching the device."""
import ctypes
import os
import re

import pytest

import device_draft_verification_specverify_amd as sv

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "specverify.h")

pytestmark = pytest.mark.skipif(not os.path.exists(sv.LIBRARY),
                                reason="libspecverify.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(specverify_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = sv.load_library()
    names = declared_functions()
    assert set(names) == {"specverify_workspace_size", "specverify_normalize", "specverify_accept",
                          "specverify_residual_sample", "specverify_step",
                          "specverify_step_noalloc",
                          "specverify_accept_prob_workspace_size", "specverify_accept_prob",
                          "specverify_geometric_fanout", "specverify_residual_topf",
                          "specverify_cache_lookup",
                          "specverify_bandit_state_size", "specverify_bandit_init",
                          "specverify_bandit_select", "specverify_bandit_update",
                          "specverify_bandit_stats", "specverify_step_reward",
                          "specverify_branch_prune",
                          "specverify_time_next_stream_kernel", "specverify_check_count",
                          "specverify_status_string", "specverify_version"}
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(sv._SIGNATURES)


def test_version_and_status_strings():
    lib = sv.load_library()
    assert lib.specverify_version() >= 100
    for code in (0, -1, -2, -3, -4, -5, 99):
        assert lib.specverify_status_string(code)


def test_timing_hook_needs_both_events_or_neither():
    lib = sv.load_library()
    assert lib.specverify_time_next_stream_kernel(8, None) == -1
    assert lib.specverify_time_next_stream_kernel(None, 8) == -1
    assert lib.specverify_time_next_stream_kernel(None, None) == 0   # clears


def test_check_count_needs_the_checked_build():
    lib = sv.load_library()
    n = ctypes.c_uint32(7)
    if os.path.basename(sv.LIBRARY) == "libspecverify.so":
        assert lib.specverify_check_count(ctypes.byref(n), 0) == sv.SV_ENOCHECKS
        assert sv.check_count() is None


def test_workspace_sizes():
    lib = sv.load_library()
    c3 = lib.specverify_workspace_size(64, 1, 8, 128256, 1)
    assert c3 > 0 and c3 % 256 == 0
    assert lib.specverify_workspace_size(512, 4, 8, 128256, 1) > c3
    assert lib.specverify_workspace_size(64, 0, 8, 128256, 1) > 0          # normalize layout
    for bad in ((0, 1, 8, 100, 1), (4, 1, 33, 100, 1), (4, 3, 22, 100, 1), (4, 1, 8, 0, 1),
                (4, 1, 8, 100, 7), (4, 1, 8, 2 ** 31, 1)):
        assert lib.specverify_workspace_size(*bad) == 0, bad


def _step(lib, **over):
    a = dict(t=8, d=8, dtype=1, tok=8, B=2, K=1, g=4, V=1000, tsb=5000, tsj=1000, dsb=4000, dsk=4000,
             dsj=1000, T=8, seed=1, pos0=None, n=8, y=8, lp=None, lq=None, zt=None, zd=None,
             err=None, ws=256, wsb=1 << 24, st=None)
    a.update(over)
    order = ["t", "d", "dtype", "tok", "B", "K", "g", "V", "tsb", "tsj", "dsb", "dsk", "dsj", "T",
             "seed", "pos0", "n", "y", "lp", "lq", "zt", "zd", "err", "ws", "wsb", "st"]
    return lib.specverify_step(*[a[k] for k in order])


def test_step_argument_validation_happens_on_the_host():
    # Fake device pointers: every call below must be rejected before any HIP call.
    lib = sv.load_library()
    assert _step(lib, t=None) == -1
    assert _step(lib, tok=None) == -1
    assert _step(lib, n=None) == -1
    assert _step(lib, B=0) == -1
    assert _step(lib, g=0) == -1
    assert _step(lib, g=33) == -1
    assert _step(lib, K=3, g=22) == -1            # K * gamma > 64
    assert _step(lib, V=0) == -1
    assert _step(lib, V=2 ** 31) == -1
    assert _step(lib, tsb=-1) == -1
    assert _step(lib, dtype=5) == -2
    assert _step(lib, ws=None) == -3
    need = lib.specverify_workspace_size(2, 1, 4, 1000, 1)
    assert _step(lib, wsb=need - 1) == -3
    assert _step(lib, ws=264) == -4                # misaligned workspace


def test_other_entry_points_validate_on_the_host():
    lib = sv.load_library()
    assert lib.specverify_normalize(None, 1, 2, 3, 100, 300, 100, 8, 8, None, 256, 1 << 20, None) == -1
    assert lib.specverify_normalize(8, 9, 2, 3, 100, 300, 100, 8, 8, None, 256, 1 << 20, None) == -2
    assert lib.specverify_normalize(8, 1, 2, 3, 100, 300, 100, 8, 8, None, 256, 16, None) == -3
    # 2^31 or more 8 KB chunks in one call (over 16 TiB of rows): rejected before any HIP call
    assert lib.specverify_normalize(8, 1, 2 ** 27, 1, 2 ** 20, 0, 0, 8, 8, None, 256, 1 << 20,
                                    None) == -1
    assert lib.specverify_accept(None, 8, 2, 1, 4, 0, None, 8, None, None) == -1
    assert lib.specverify_accept(8, 8, 2, 1, 33, 0, None, 8, None, None) == -1
    assert lib.specverify_accept(8, 8, 0, 1, 4, 0, None, 8, None, None) == -1
    args = [8, 8, 1, 2, 1, 4, 1000, 5000, 1000, 4000, 4000, 1000, 8, 8, 8, 8, 8, 1, None, 8, 256,
            1 << 24, None]
    bad = list(args)
    bad[15] = None                                  # accept_len
    assert lib.specverify_residual_sample(*bad) == -1
    bad = list(args)
    bad[2] = 3
    assert lib.specverify_residual_sample(*bad) == -2
    bad = list(args)
    bad[20] = None
    assert lib.specverify_residual_sample(*bad) == -3


def test_accept_prob_validates_on_the_host():
    lib = sv.load_library()
    need = lib.specverify_accept_prob_workspace_size(2, 1, 4, 1000, 1)
    assert lib.specverify_accept_prob_workspace_size(64, 1, 8, 128256, 1) > need > 0
    assert lib.specverify_accept_prob_workspace_size(2, 1, 33, 1000, 1) == 0
    assert lib.specverify_accept_prob_workspace_size(2, 1, 4, 1000, 7) == 0
    # target, draft, dtype, B, K, gamma, V, 5 strides, T, lnZ_t, lnZ_d, alpha, law, ws, bytes, stream
    args = [8, 8, 1, 2, 1, 4, 1000, 5000, 1000, 4000, 4000, 1000, 8, 8, 8, 8, None, 256, need, None]
    for i, code in ((0, -1), (12, -1), (13, -1), (14, -1), (15, -1)):
        bad = list(args)
        bad[i] = None
        assert lib.specverify_accept_prob(*bad) == code, i
    bad = list(args)
    bad[2] = 4
    assert lib.specverify_accept_prob(*bad) == -2
    bad = list(args)
    bad[7] = -1
    assert lib.specverify_accept_prob(*bad) == -1
    bad = list(args)
    bad[5] = 0
    assert lib.specverify_accept_prob(*bad) == -1
    bad = list(args)
    bad[18] = need - 1
    assert lib.specverify_accept_prob(*bad) == -3
    bad = list(args)
    bad[17] = 264
    assert lib.specverify_accept_prob(*bad) == -4


def test_geometric_fanout_matches_the_oracle():
    # a pure host function: checked against the oracle here, without a GPU
    import oracle
    for g, tot, a in ((2, 7, 0.5), (2, 10, 0.5), (3, 6, 1.0), (8, 64, 0.6), (4, 33, 0.9),
                      (1, 5, 0.2), (32, 300, 0.85), (8, 0, 0.5), (5, 384, 1.0)):
        assert sv.geometric_fanout(g, tot, a) == oracle.geometric_fanout(g, tot, a).tolist(), (g, tot, a)
    lib = sv.load_library()
    import ctypes
    out = (ctypes.c_int32 * 40)()
    assert lib.specverify_geometric_fanout(2, 10, 0.0, out) == -1
    assert lib.specverify_geometric_fanout(2, 10, 1.5, out) == -1
    assert lib.specverify_geometric_fanout(33, 10, 0.5, out) == -1
    assert lib.specverify_geometric_fanout(2, 3 * 64 + 1, 1.0, out) == -1
    assert lib.specverify_geometric_fanout(2, 10, 0.5, None) == -1


def test_topf_and_lookup_validate_on_the_host():
    import ctypes
    lib = sv.load_library()
    fan = (ctypes.c_int32 * 5)(4, 3, 2, 1, 1)
    args = [8, 8, 1, 2, 1, 4, 1000, 5000, 1000, 4000, 4000, 1000, 8, 8, 8, fan, 8, None, None]
    for i in (0, 12, 13, 14, 15, 16):
        bad = list(args)
        bad[i] = None
        assert lib.specverify_residual_topf(*bad) == -1, i
    bad = list(args)
    bad[2] = 7
    assert lib.specverify_residual_topf(*bad) == -2
    bad = list(args)
    bad[15] = (ctypes.c_int32 * 5)(4, 65, 2, 1, 1)
    assert lib.specverify_residual_topf(*bad) == -1
    bad = list(args)
    bad[15] = (ctypes.c_int32 * 5)(4, -1, 2, 1, 1)
    assert lib.specverify_residual_topf(*bad) == -1
    bad = list(args)
    bad[10] = -3
    assert lib.specverify_residual_topf(*bad) == -1
    largs = [8, fan, 2, 1, 4, 8, 8, 8, None]
    for i in (0, 1, 5, 6, 7):
        bad = list(largs)
        bad[i] = None
        assert lib.specverify_cache_lookup(*bad) == -1, i
    bad = list(largs)
    bad[4] = 0
    assert lib.specverify_cache_lookup(*bad) == -1


def test_branch_prune_validates_on_the_host():
    lib = sv.load_library()
    args = [8, 4, 2, 8, -1.0, 1, 8, None, None, None]
    bad = list(args); bad[0] = None
    assert lib.specverify_branch_prune(*bad) == -1
    bad = list(args); bad[6] = None
    assert lib.specverify_branch_prune(*bad) == -1
    bad = list(args); bad[2] = 9            # K * gamma > 64
    assert lib.specverify_branch_prune(*bad) == -1
    bad = list(args); bad[5] = -1
    assert lib.specverify_branch_prune(*bad) == -1
    bad = list(args); bad[4] = float("nan")
    assert lib.specverify_branch_prune(*bad) == -1


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(sv.SpecVerifyError):
        sv.specverify_normalize(torch.zeros(1, 2, 8), torch.ones(1))


def test_noalloc_step_refuses_sizes_beyond_its_scratch_on_the_host():
    # the size check comes before any device call: the pointers are never touched
    lib = sv.load_library()
    fake = ctypes.c_void_p(0x1000)
    B, K, g, V = 2048, 4, 8, 128256
    assert sv.workspace_size(B, K, g, V, sv.SV_BF16) > sv.NOALLOC_SCRATCH_BYTES
    st = lib.specverify_step_noalloc(fake, fake, sv.SV_BF16, fake, B, K, g, V, (g + 1) * V, V,
                                     K * g * V, g * V, V, fake, 1, None, fake, fake, None, None,
                                     None, None, None, None)
    assert st == sv.SV_ESCRATCH
    assert b"SV_NOALLOC_SCRATCH_BYTES" in lib.specverify_status_string(st)
    # argument errors are reported first, as by specverify_step
    assert lib.specverify_step_noalloc(None, fake, sv.SV_BF16, fake, B, K, g, V, 0, 0, 0, 0, 0,
                                       fake, 1, None, fake, fake, None, None, None, None, None,
                                       None) == -1  # SV_EINVAL
