"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/sanitized_host_driver.cpp is linked against a build of the library's
sources whose host side is instrumented (hipcc's -Xarch_host places each
sanitizer on the host pass only; the device code, never run here, is built at
-O0 to keep the compile short). The driver calls every GPU entry point with
arguments the host checks refuse (no HIP call is made) and runs the pure host
functions; any sanitizer report aborts it. The selector's picks under the
driver's fixed reward function must equal the oracle's.
"""
import os
import re
import shutil
import subprocess

import pytest

from oracle import bandit as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "device_draft_verification_specverify_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
ROCM_LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(HIPCC))), "lib")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def reward_of(step: int, arm: int) -> float:
    return ((step * 7 + arm * 13) % 17) / 16.0


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(HIPCC) or shutil.which("g++") is None:
        pytest.skip("hipcc or g++ missing")
    d = tmp_path_factory.mktemp("san")
    inc = ["-I", os.path.join(ROOT, "include")]
    lib_o, drv_o, bandit_o, exe = (str(d / n) for n in ("sv.o", "drv.o", "bandit.o", "drv"))
    host_san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    steps = [
        [HIPCC, "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xarch_device", "-O0",
         "-Xarch_host", "-O1", *SAN, *inc, "-c", os.path.join(SRC, "specverify.hip"), "-o", lib_o],
        ["g++", "-O1", "-g", "-std=c++17", *host_san, *inc, "-c", os.path.join(SRC, "bandit.cpp"),
         "-o", bandit_o],
        ["g++", "-O1", "-g", "-std=c++17", *host_san, *inc, "-c",
         os.path.join(ROOT, "tests", "sanitized_host_driver.cpp"), "-o", drv_o],
        ["g++", *host_san, lib_o, bandit_o, drv_o, f"-L{ROCM_LIB}", "-lamdhip64",
         f"-Wl,-rpath,{ROCM_LIB}", "-o", exe],
    ]
    for cmd in steps:
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-3000:]
    return exe


def test_host_code_is_clean_under_sanitizers_and_picks_match_the_oracle(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=120)
    assert "ERROR: AddressSanitizer" not in res.stderr, res.stderr[-3000:]
    assert "runtime error" not in res.stderr, res.stderr[-3000:]
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    picks = re.findall(r"^picks (\d+) (\d+) (\d+):((?: \d+)+)$", res.stdout, re.M)
    assert len(picks) == 4
    for policy, arms, seed, seq in picks:
        got = [int(x) for x in seq.split()]
        ora = bd.Bandit(int(arms), int(policy), seed=int(seed))
        want = []
        for s in range(len(got)):
            a = ora.select()
            want.append(a)
            ora.update(a, reward_of(s, a))
        assert got == want, (policy, arms, seed)
