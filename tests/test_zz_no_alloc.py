"""The gate entry point that allocates nothing (tg_gate_score_prepacked_noalloc) against the workspace entry
point it mirrors (tg_gate_score_prepacked), through the C ABI: bit-identical scores on two calls in a row, the
second with a smaller input (the library's scratch keeps the first call's contents), and the size limit."""
import ctypes
import sys

import numpy as np
import pytest

from _lib import binding
from learned_token_pruning_amd import workloads as W


def _say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def _inputs(tg, torch, n_tokens, docs, seed):
    """A packed batch: prompt i has docs[i] document tokens after a 16-token request and before 48 question
    tokens; d = 2048, h = 256, N(0,1) hidden rows, Xavier-normal W1 and w2."""
    rng = np.random.default_rng(seed)
    lens = [16 + nd + 48 for nd in docs]
    offs = np.concatenate([[0], np.cumsum(lens)]).tolist()
    assert offs[-1] == n_tokens
    plan = tg.plan_segments(offs, [16] * len(docs), [16 + nd for nd in docs], [1 << 30] * len(docs), device="cuda")
    d, h = 2048, 256
    x = W.f32_to_bf16_bits(rng.standard_normal((n_tokens, d)).astype(np.float32))
    w1 = W.f32_to_bf16_bits((rng.standard_normal((h, d)) * np.sqrt(2.0 / (d + h))).astype(np.float32))
    w2 = (rng.standard_normal(h) * np.sqrt(2.0 / (h + 1))).astype(np.float32)
    dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    return plan, dev(x), dev(w1), torch.from_numpy(w2).cuda(), h


@pytest.mark.gpu
def test_noalloc_gate_equals_workspace_gate_twice():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tg = binding()
    for call, docs in enumerate(([20000, 3000, 9000], [700, 1200])):
        n = sum(16 + nd + 48 for nd in docs)
        _say("no-alloc gate call", call, "prompts", docs)
        plan, x, w1, w2, h = _inputs(tg, torch, n, docs, seed=100 + call)
        w1p = tg.gate_pack_w1(w1)
        ref = tg.gate_score_prepacked(x, w1p, h, None, w2, 0.0, plan)
        got = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
        tg.gate_score_prepacked_noalloc(x, w1p, h, None, w2, 0.0, plan, got)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), f"call {call}: scores differ"


@pytest.mark.gpu
def test_noalloc_gate_rejects_plans_past_its_scratch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tg = binding()
    cap = tg.gate_noalloc_max_tiles()
    assert cap == (512 << 10) // 8
    # one prompt whose document needs one 64-row tile more than the scratch holds
    nd = cap * 64 + 1
    plan = tg.plan_segments([0, nd], [0], [nd], [0], device="cuda")
    L = tg._lib
    st = L.tg_gate_score_prepacked_noalloc(ctypes.c_void_p(0x1000), 2048, 2048, ctypes.c_void_p(0x1000), None,
                                           ctypes.c_void_p(0x1000), 0.0, 256, tg._dev_table(plan),
                                           ctypes.byref(plan.info), 1e-6, ctypes.c_void_p(0x1000), None)
    assert st == -3  # TG_ERR_WORKSPACE, before anything touches the (fake) pointers
