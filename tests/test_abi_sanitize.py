"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU needed).

Every HIP source is compiled again with the sanitizers on its host side only (device code is unchanged) and
linked with tests/abi_sanitize_check.cpp, which calls every entry point with exact-size heap arrays: random
segment tables through tg_plan_segments (checked against their totals), invalid tables, every attention, gate,
select, decoder-layer, compaction, dense and decode entry point on fake device pointers, and the workspace
sizing functions over wide shape ranges.  Without a device every call ends at validation or at the device
check, so the code covered is argument validation, planning and sizing; an out-of-bounds host access, a
signed overflow or a bad shift aborts the program."""
import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from _lib import ROOT

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    out = tmp_path_factory.mktemp("abi_sanitize")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "learned_token_pruning_amd", "csrc")]
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    srcs = sorted(glob.glob(os.path.join(ROOT, "learned_token_pruning_amd", "csrc", "*.hip")))
    jobs = [[hipcc, "-std=c++17", "-O1", "-g", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", *SAN_HOST, *inc, "-c", s, "-o", str(out / (os.path.basename(s) + ".o"))]
            for s in srcs]
    jobs.append([hipcc, "-std=c++17", "-O1", "-g", "-x", "hip", "--cuda-host-only", *SAN_HOST, *inc, "-c",
                 os.path.join(ROOT, "tests", "abi_sanitize_check.cpp"), "-o", str(out / "check.o")])

    def run(cmd):
        return subprocess.run(cmd, capture_output=True, text=True)

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        for r in ex.map(run, jobs):
            assert r.returncode == 0, r.stdout + r.stderr
    exe = str(out / "abi_check")
    objs = [j[-1] for j in jobs]
    r = run([os.path.join(ROCM, "llvm", "bin", "clang++"), "-fsanitize=address,undefined", *objs,
             "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe])
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


@pytest.mark.parametrize("seed", [1, 2])
def test_abi_host_code_is_sanitizer_clean(checker, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([checker, "2000", str(seed)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.stdout + r.stderr)[-4000:]
