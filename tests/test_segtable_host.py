"""The segment-table clamp, on the host: every kernel reads its prompt's entry through SegTable::clamp
(csrc/common.h) with the totals the host validated, so a device table that disagrees with its info cannot move
an access outside the arrays sized from that info.  A random fuzz checks that every clamped entry lies inside
the totals; tables built by tg_plan_segments must pass through unchanged (no GPU needed)."""
import os
import subprocess

import numpy as np
import pytest

from _lib import ROOT, binding
from learned_token_pruning_amd import workloads as W

tg = binding()


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("segtable") / "segtable_check")
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    cmd = [hipcc, "-std=c++17", "-O2", "-x", "hip", "--cuda-host-only", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "learned_token_pruning_amd", "csrc"),
           os.path.join(ROOT, "tests", "segtable_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_clamped_entries_stay_inside_the_totals(checker, seed):
    r = subprocess.run([checker, "fuzz", "300000", str(seed)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


def _tables():
    rng = np.random.default_rng(5)
    out = []
    for n_seg, max_len in ((40, 4096), (8, 40000)):
        s = W.random_segments(rng, n_seg, max_len)
        out.append((s.seg_start, s.doc_begin, s.doc_end, s.k_budget))
    for _ in range(20):
        n_seg = int(rng.integers(1, 40))
        lens = rng.integers(0, 5000, n_seg)
        starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        b = np.array([int(rng.integers(0, ln + 1)) for ln in lens])
        e = np.array([int(rng.integers(bb, ln + 1)) for bb, ln in zip(b, lens)])
        k = rng.integers(0, 6000, n_seg)
        out.append((starts.tolist(), b.tolist(), e.tolist(), k.tolist()))
    out.append(([0, 65536], [0], [65472], [4096]))
    out.append(([0, 0, 5], [0, 0], [0, 5], [0, 0]))  # an empty prompt and a zero budget
    return out


def test_planned_tables_pass_unchanged(checker):
    for seg_start, doc_begin, doc_end, k in _tables():
        plan = tg.plan_segments(seg_start, doc_begin, doc_end, k, None)
        i = plan.info
        lines = [f"{i.n_tokens} {i.total_kept} {i.max_seg_len} {i.max_doc_len} {i.max_kept_len} {plan.table.shape[0]}"]
        lines += [" ".join(str(int(v)) for v in row[:7]) for row in plan.table]
        r = subprocess.run([checker, "identity"], input="\n".join(lines) + "\n", capture_output=True, text=True,
                           timeout=60)
        assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
