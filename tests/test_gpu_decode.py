"""Parity of the decode step (tg_gated_attention_decode, through the C ABI)
with the oracle: max |d| <= 2e-2 on the bf16 outputs, on seeded inputs."""
import functools
import sys

import numpy as np
import pytest

import oracle
from _lib import binding
from learned_token_pruning_amd import workloads as W

pytestmark = pytest.mark.gpu

ATTN_ATOL = 2e-2


def _say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


@functools.lru_cache(maxsize=None)
def _tg():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return binding()


def _bf16(rng, shape, scale=1.0):
    return W.f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def run_decode(q, kc, vc, s, tau, gain, lens):
    import torch
    tg = _tg()
    dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    f32 = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    out = tg.gated_attention_decode(dev(q), dev(kc), dev(vc), f32(s), f32(tau), f32(gain),
                                    torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda())
    return W.bf16_bits_to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16))


def check(got, q, kc, vc, s, tau, gain, lens):
    f64 = W.bf16_bits_to_f64
    ref = oracle.gated_attention_decode(f64(q), f64(kc), f64(vc), None if s is None else s.astype(np.float64),
                                        None if tau is None else tau.astype(np.float64),
                                        None if gain is None else gain.astype(np.float64), lens)
    err = np.abs(got - ref).max()
    assert err <= ATTN_ATOL, f"max abs err {err:.3e}"
    return err


@pytest.mark.parametrize("d,hq,hkv", [(128, 16, 8), (128, 16, 4), (128, 8, 8), (64, 4, 2), (64, 8, 2), (64, 2, 2)])
def test_decode_ragged_lengths(d, hq, hkv):
    _say("decode ragged", d, hq, hkv)
    rng = np.random.default_rng(d + 3 * hq + hkv)
    lens = [0, 1, 63, 255, 256, 257, 700, 2112]
    b, cap = len(lens), 2200
    q = _bf16(rng, (b, hq, d))
    kc, vc = _bf16(rng, (b, cap, hkv, d)), _bf16(rng, (b, cap, hkv, d))
    s = rng.standard_normal((b, cap)).astype(np.float32)
    tau = rng.uniform(0.8, 1.2, hq).astype(np.float32)
    gain = rng.uniform(0.5, 1.5, hq).astype(np.float32)
    check(run_decode(q, kc, vc, s, tau, gain, lens), q, kc, vc, s, tau, gain, lens)
    check(run_decode(q, kc, vc, None, None, None, lens), q, kc, vc, None, None, None, lens)
    # a temperature per query (sequence, head)
    tq = rng.uniform(0.2, 1.5, (b, hq)).astype(np.float32)
    check(run_decode(q, kc, vc, s, tq, gain, lens), q, kc, vc, s, tq, gain, lens)


def test_decode_lengths_are_clamped():
    _say("decode clamped lengths")
    rng = np.random.default_rng(5)
    b, cap, hq, hkv, d = 3, 300, 4, 2, 64
    q = _bf16(rng, (b, hq, d))
    kc, vc = _bf16(rng, (b, cap, hkv, d)), _bf16(rng, (b, cap, hkv, d))
    s = rng.standard_normal((b, cap)).astype(np.float32)
    got = run_decode(q, kc, vc, s, None, np.ones(hq, np.float32), [-5, cap + 100, 17])
    check(got, q, kc, vc, s, None, np.ones(hq, np.float32), [0, cap, 17])


def test_decode_over_pruned_cache_matches_prefill_last_row():
    """Workload 2 pruned to K = 2048: the cache holds the 2112 kept rows plus
    one generated token (score 0).  The decode step matches the oracle, and a
    decode of the last kept row over the kept rows matches the prefill
    kernel's last output row within the same tolerance."""
    import torch
    _say("decode over the workload-2 pruned cache")
    tg = _tg()
    L = W.workload(2)
    s = W.mixture_scores(2, L.segments)
    seg = L.segments.with_budget(2048)
    kept, offs = oracle.kept_indices(s, seg.seg_start, seg.doc_begin, seg.doc_end, seg.k_budget)
    m = kept.size
    assert m == 2112
    rng = np.random.default_rng(9)
    kq, kk, kv = (oracle.compact_rows(t, kept) for t in (L.q, L.k, L.v))
    ks = oracle.compact_rows(s, kept).astype(np.float32)
    hq, hkv, d = kq.shape[1], kk.shape[1], kk.shape[2]
    cap = m + 1
    kc = np.concatenate([kk, _bf16(rng, (1, hkv, d))])[None]
    vc = np.concatenate([kv, _bf16(rng, (1, hkv, d))])[None]
    sc = np.concatenate([ks, [0.0]]).astype(np.float32)[None]
    qn = _bf16(rng, (1, hq, d))
    check(run_decode(qn, kc, vc, sc, L.tau, L.gain, [cap]), qn, kc, vc, sc, L.tau, L.gain, [cap])
    # the last kept row, decoded over the kept rows only, against the prefill kernel
    got = run_decode(kq[m - 1:m], kc, vc, sc, L.tau, L.gain, [m])
    plan = tg.plan_segments([0, m], [0], [0], [0], device="cuda")
    dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    pre = tg.gated_attention_prefill(dev(kq), dev(kk), dev(kv), f32(ks), f32(L.tau), f32(L.gain), plan)
    last = W.bf16_bits_to_f64(pre[m - 1].view(torch.int16).cpu().numpy().view(np.uint16))
    assert np.abs(got[0] - last).max() <= ATTN_ATOL


def test_decode_long_cache():
    _say("decode long cache")
    rng = np.random.default_rng(13)
    b, cap, hq, hkv, d = 2, 33000, 16, 8, 128
    q = _bf16(rng, (b, hq, d))
    kc, vc = _bf16(rng, (b, cap, hkv, d)), _bf16(rng, (b, cap, hkv, d))
    s = rng.standard_normal((b, cap)).astype(np.float32)
    tau = rng.uniform(0.8, 1.2, hq).astype(np.float32)
    gain = rng.uniform(0.5, 1.5, hq).astype(np.float32)
    lens = [cap, 32769]
    check(run_decode(q, kc, vc, s, tau, gain, lens), q, kc, vc, s, tau, gain, lens)


def test_decode_deterministic():
    _say("decode determinism")
    rng = np.random.default_rng(14)
    b, cap, hq, hkv, d = 4, 1000, 16, 8, 128
    q = _bf16(rng, (b, hq, d))
    kc, vc = _bf16(rng, (b, cap, hkv, d)), _bf16(rng, (b, cap, hkv, d))
    s = rng.standard_normal((b, cap)).astype(np.float32)
    g = np.ones(hq, np.float32)
    a = run_decode(q, kc, vc, s, None, g, [1000, 999, 3, 512])
    c = run_decode(q, kc, vc, s, None, g, [1000, 999, 3, 512])
    assert a.tobytes() == c.tobytes()
