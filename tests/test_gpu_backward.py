"""Parity of the attention backward (tg_gated_attention_prefill_lse and
tg_gated_attention_backward, through the C ABI) with the oracle.

Bar: the saved log-sum-exp within 4e-3 absolute (the forward's denominator
sums bf16-rounded probabilities, each within a relative 2^-9, so the sum and
thus exp(lse) are within a relative 2^-8 and lse within ln(1 + 2^-8)); every
gradient within
GRAD_RTOL of the largest magnitude of its oracle tensor (max-norm relative
error).  The products run on bf16 operands (P and dZ are rounded to bf16,
relative error 2^-9 each) with fp32 accumulation, and the forward output the
backward reads is itself bf16, so errors of a few 1e-3 of the tensor's scale
are expected; 2e-2 leaves margin without hiding a wrong term (a dropped or
mis-signed term is an O(1) relative error)."""
import functools
import sys

import numpy as np
import pytest

import oracle
from _lib import binding
from learned_token_pruning_amd import workloads as W

pytestmark = pytest.mark.gpu

GRAD_RTOL = 2e-2
LSE_ATOL = 4e-3


def _say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


@functools.lru_cache(maxsize=None)
def _tg():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return binding()


def _dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _dev_f32(a):
    import torch
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def run_backward(q, k, v, s, tau, gain, offs, dout):
    import torch
    tg = _tg()
    n_seg = len(offs) - 1
    plan = tg.plan_segments(list(offs), [0] * n_seg, [0] * n_seg, [0] * n_seg, device="cuda")
    qd, kd, vd = _dev_bf16(q), _dev_bf16(k), _dev_bf16(v)
    sd, td, gd = _dev_f32(s), _dev_f32(tau), _dev_f32(gain)
    out, lse = tg.gated_attention_prefill_lse(qd, kd, vd, sd, td, gd, plan)
    g = tg.gated_attention_backward(qd, kd, vd, sd, td, gd, plan, out, _dev_bf16(dout), lse)
    torch.cuda.synchronize()
    res = {name: t.cpu().numpy().astype(np.float64) for name, t in g.items()}
    res["lse"] = lse.cpu().numpy().astype(np.float64)
    return res


def check_backward(got, q, k, v, s, tau, gain, offs, dout):
    f64 = W.bf16_bits_to_f64
    s64 = None if s is None else s.astype(np.float64)
    t64 = None if tau is None else tau.astype(np.float64)
    g64 = None if gain is None else gain.astype(np.float64)
    ref = oracle.gated_attention_backward(f64(q), f64(k), f64(v), s64, t64, g64, offs, f64(dout))
    lse = oracle.attention_logsumexp(f64(q), f64(k), s64, t64, g64, offs)
    assert np.abs(got["lse"] - lse).max() <= LSE_ATOL
    errs = {}
    for name in ("dq", "dk", "dv", "ds", "dgain", "dtau"):
        scale = max(np.abs(ref[name]).max(), 1e-30)
        errs[name] = np.abs(got[name] - ref[name]).max() / scale
        if np.abs(ref[name]).max() == 0.0:
            assert np.abs(got[name]).max() == 0.0, name
        else:
            assert errs[name] <= GRAD_RTOL, f"{name}: relative max error {errs[name]:.3e}"
    return errs


def _inputs(rng, m, hq, hkv, d):
    q = W.f32_to_bf16_bits(rng.standard_normal((m, hq, d)).astype(np.float32))
    k = W.f32_to_bf16_bits(rng.standard_normal((m, hkv, d)).astype(np.float32))
    v = W.f32_to_bf16_bits(rng.standard_normal((m, hkv, d)).astype(np.float32))
    dout = W.f32_to_bf16_bits(rng.standard_normal((m, hq, d)).astype(np.float32))
    s = rng.standard_normal(m).astype(np.float32)
    tau = rng.uniform(0.8, 1.2, hq).astype(np.float32)
    gain = rng.uniform(0.5, 1.5, hq).astype(np.float32)
    return q, k, v, dout, s, tau, gain


@pytest.mark.parametrize("d,hq,hkv", [(64, 4, 2), (64, 4, 4), (64, 8, 2), (128, 2, 2), (128, 8, 4), (128, 16, 8),
                                     (128, 16, 4)])
def test_backward_ragged(d, hq, hkv):
    _say("backward ragged", d, hq, hkv)
    rng = np.random.default_rng(d + 5 * hq + hkv)
    lens = [1, 63, 64, 65, 130, 0, 257]
    offs = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, dout, s, tau, gain = _inputs(rng, int(offs[-1]), hq, hkv, d)
    tau[0] = -tau[0]  # a negative temperature
    check_backward(run_backward(q, k, v, s, tau, gain, offs, dout), q, k, v, s, tau, gain, offs, dout)
    got = run_backward(q, k, v, None, None, None, offs, dout)
    check_backward(got, q, k, v, None, None, None, offs, dout)


def test_backward_workload_2_kept_rows():
    """The 2112 kept rows of workload 2 (16 Q / 8 KV heads, D = 128) with
    their gate scores as the bias, against the oracle at full size."""
    _say("backward workload 2")
    L = W.workload(2)
    s = W.mixture_scores(2, L.segments)
    seg = L.segments.with_budget(2048)
    kept, offs = oracle.kept_indices(s, seg.seg_start, seg.doc_begin, seg.doc_end, seg.k_budget)
    q, k, v = (oracle.compact_rows(t, kept) for t in (L.q, L.k, L.v))
    sc = oracle.compact_rows(s, kept).astype(np.float32)
    rng = np.random.default_rng(41)
    dout = W.f32_to_bf16_bits(rng.standard_normal(q.shape).astype(np.float32))
    got = run_backward(q, k, v, sc, L.tau, L.gain, offs, dout)
    check_backward(got, q, k, v, sc, L.tau, L.gain, offs, dout)


def test_backward_deterministic():
    _say("backward determinism")
    rng = np.random.default_rng(42)
    offs = [0, 300, 301, 700]
    q, k, v, dout, s, tau, gain = _inputs(rng, 700, 16, 8, 128)
    a = run_backward(q, k, v, s, tau, gain, offs, dout)
    b = run_backward(q, k, v, s, tau, gain, offs, dout)
    for name in a:
        assert a[name].tobytes() == b[name].tobytes(), name


def test_backward_empty_plan():
    import torch
    tg = _tg()
    plan = tg.plan_segments([0, 0], [0], [0], [0], device="cuda")
    e = torch.empty((0, 4, 64), dtype=torch.bfloat16, device="cuda")
    e2 = torch.empty((0, 2, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((0, 4), dtype=torch.float32, device="cuda")
    g = tg.gated_attention_backward(e, e2, e2, None, None, None, plan, e, e, lse)
    torch.cuda.synchronize()
    assert g["dgain"].abs().max().item() == 0.0 and g["dtau"].abs().max().item() == 0.0
