"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Indices and compaction: bit-exact.  Gate scores: |d| <= 1e-3 * max(|ref|, rms(ref))
per element.  Attention: max |d| <= 2e-2 on the bf16 outputs.  Inputs come
from the seeded generators only; expected values only from the oracle.
"""
import functools
import sys

import numpy as np
import pytest

import oracle
from _lib import binding
from learned_token_pruning_amd import workloads as W

pytestmark = pytest.mark.gpu

SCORE_RTOL = 1e-3
ATTN_ATOL = 2e-2


def _say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


@functools.lru_cache(maxsize=None)
def _tg():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return binding()


def dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_f32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host_bf16(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def f64(bits):
    return W.bf16_bits_to_f64(bits)


@functools.lru_cache(maxsize=None)
def layer(idx, with_qkv=True):
    return W.workload(idx, with_qkv=with_qkv)


def check_scores(got, ref, doc_mask):
    got = np.asarray(got, dtype=np.float64)
    assert np.all(got[~doc_mask] == 0.0), "non-document scores must be exactly 0"
    if doc_mask.any():
        r = ref[doc_mask]
        floor = max(np.sqrt(np.mean(r * r)), 1e-30)
        err = np.abs(got[doc_mask] - r) / np.maximum(np.abs(r), floor)
        assert err.max() <= SCORE_RTOL, f"max rel err {err.max():.3e}"


def doc_mask_of(seg):
    m = np.zeros(seg.n_tokens, bool)
    for i in range(seg.n_seg):
        m[seg.seg_start[i] + seg.doc_begin[i]: seg.seg_start[i] + seg.doc_end[i]] = True
    return m


def run_gate(L, eps=1e-6, b1=None, b2=0.0):
    tg = _tg()
    plan = tg.plan_from(L.segments, device="cuda")
    s = tg.gate_score(dev_bf16(L.x), dev_bf16(L.w1), None if b1 is None else dev_f32(b1), dev_f32(L.w2), b2, plan,
                      rms_eps=eps)
    return s.cpu().numpy()


def oracle_gate(L, eps=1e-6, b1=None, b2=0.0):
    seg = L.segments
    return oracle.gate_scores(f64(L.x), f64(L.w1), b1, L.w2.astype(np.float64), b2, seg.seg_start, seg.doc_begin,
                              seg.doc_end, eps)


# ----------------------------------------------------------------------------- gate


@pytest.mark.parametrize("idx", [1, 2, 3])
def test_gate_workload(idx):
    _say("gate workload", idx)
    L = layer(idx, with_qkv=False)
    got = run_gate(L)
    check_scores(got, oracle_gate(L), doc_mask_of(L.segments))


def test_gate_workload_4_full_size():
    _say("gate workload 4 (N=131072)")
    L = layer(4, with_qkv=False)
    got = run_gate(L)
    check_scores(got, oracle_gate(L), doc_mask_of(L.segments))


@pytest.mark.parametrize("h,d", [(64, 128), (128, 64), (192, 256), (256, 192)])
def test_gate_ragged_segments(h, d):
    _say("gate ragged", h, d)
    rng = np.random.default_rng(h + d)
    seg = W.random_segments(rng, 7, 300)
    seg.doc_begin[2], seg.doc_end[2] = 0, 0  # an empty document
    L = W.make_gated_layer(11, seg, d, h, 2, 1, 64, with_qkv=False)
    b1 = rng.standard_normal(h).astype(np.float32) * 0.1
    got = run_gate(L, b1=b1, b2=0.3)
    check_scores(got, oracle_gate(L, b1=b1, b2=0.3), doc_mask_of(seg))
    got_raw = run_gate(L, eps=-1.0, b1=b1, b2=0.3)
    check_scores(got_raw, oracle_gate(L, eps=-1.0, b1=b1, b2=0.3), doc_mask_of(seg))


def test_gate_ragged_large_batch():
    """A packed batch of five prompts (73K tokens): ragged document spans,
    partial last tiles, an empty document."""
    _say("gate ragged, large batch")
    rng = np.random.default_rng(77)
    lens = [17000, 16500, 9000, 30000, 600]
    starts = [0]
    for n in lens:
        starts.append(starts[-1] + n)
    db = [3, 0, 100, 0, 50]
    de = [16990, 16500, 8977, 29937, 50]  # the last prompt has an empty document
    seg = W.Segments(starts, db, de, [10, 20, 30, 40, 0])
    L = W.make_gated_layer(78, seg, 256, 128, 2, 1, 64, with_qkv=False)
    b1 = rng.standard_normal(128).astype(np.float32) * 0.1
    got = run_gate(L, b1=b1, b2=0.1)
    check_scores(got, oracle_gate(L, b1=b1, b2=0.1), doc_mask_of(seg))


@pytest.mark.parametrize("idx", [1, 2])
def test_gate_prepacked_equals_gate(idx):
    """W1 packed once (tg_gate_pack_w1) gives tg_gate_score's scores bit for bit."""
    import torch
    _say("gate prepacked", idx)
    tg = _tg()
    L = layer(idx, with_qkv=False)
    plan = tg.plan_from(L.segments, device="cuda")
    x, w1, w2 = dev_bf16(L.x), dev_bf16(L.w1), dev_f32(L.w2)
    a = tg.gate_score(x, w1, None, w2, 0.0, plan)
    b = tg.gate_score_prepacked(x, tg.gate_pack_w1(w1), w1.shape[0], None, w2, 0.0, plan)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_gate_deterministic():
    _say("gate determinism")
    L = layer(2, with_qkv=False)
    a = run_gate(L)
    b = run_gate(L)
    assert a.tobytes() == b.tobytes()


# ----------------------------------------------------------------------------- select


def run_select(scores, seg):
    tg = _tg()
    plan = tg.plan_from(seg, device="cuda")
    idx = tg.select_topk(dev_f32(scores), plan)
    return idx.cpu().numpy().astype(np.int64), plan


def check_select(scores, seg):
    got, plan = run_select(scores, seg)
    ref, offs = oracle.kept_indices(scores, seg.seg_start, seg.doc_begin, seg.doc_end, seg.k_budget)
    assert plan.kept_offsets.tolist() == offs.tolist()
    assert got.size == ref.size
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, f"first mismatch at row {bad[:5]}: got {got[bad[:5]]} ref {ref[bad[:5]]}"


@pytest.mark.parametrize("k", [1024, 2048, 4096, 8192])
def test_select_mixture_32k(k):
    _say("select 32K mixture", k)
    seg = W.single_segment(32704, 64, k)
    s = W.mixture_scores(3, seg, k_marks=(1024, 2048, 4096, 8192))
    check_select(s, seg)


@pytest.mark.parametrize("n_doc,k", [(16320, 2048), (131008, 2048), (131008, 4096)])
def test_select_long(n_doc, k):
    _say("select", n_doc, k)
    seg = W.single_segment(n_doc, 64, k)
    s = W.mixture_scores(n_doc, seg, k_marks=(k,))
    check_select(s, seg)


@pytest.mark.parametrize("k", [0, 1, 4095, 4096, 4097, 5000, 9000])
def test_select_budget_edges(k):
    _say("select budget", k)
    seg = W.single_segment(5000, 17, k)
    s = W.mixture_scores(9, seg, k_marks=(4096,))
    check_select(s, seg)


def test_select_special_values():
    _say("select special values")
    rng = np.random.default_rng(2)
    vals = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 1.0, -1.0, 3.5, 1e-40, -1e-40], np.float32)
    s = vals[rng.integers(0, vals.size, 6000)]
    for k in (0, 1, 7, 100, 1000, 2999, 5999, 6000):
        seg = W.Segments([0, 6000], [0], [5990], [k])
        check_select(s, seg)


def test_select_all_equal():
    _say("select all equal")
    s = np.zeros(10000, np.float32)
    for k in (1, 333, 9999):
        check_select(s, W.Segments([0, 10000], [100], [10000], [k]))
    s[::2] = -0.0
    check_select(s, W.Segments([0, 10000], [0], [10000], [4321]))


@pytest.mark.parametrize("seed", [0, 1, 2, 3, 4, 5])
def test_select_ragged_segments(seed):
    """Batches of 40 prompts; seeds 3 to 5 have prompts past 16K tokens, so they run the multi-workgroup
    path next to short prompts: seed 3 on 512-token slices (40 x 5 slices of 4096 tokens would be under 256
    workgroups), seeds 4 and 5 on 4096-token slices."""
    _say("select ragged", seed)
    rng = np.random.default_rng(100 + seed)
    seg = W.random_segments(rng, 40, [50, 500, 5000, 20000, 70000, 70000][seed])
    s = W.mixture_scores(seed, seg)
    if seed in (3, 5):  # coarse values: many ties everywhere
        s = np.round(s * 2) / 2
    check_select(s.astype(np.float32), seg)


@pytest.mark.parametrize("k", [0, 1, 4095, 4096, 40000, 40003, 50000])
def test_select_budget_edges_long(k):
    """Budget edges on the multi-workgroup path (one 40003-token document)."""
    _say("select budget long", k)
    seg = W.single_segment(40003, 5, k)
    s = W.mixture_scores(11, seg, k_marks=(4096,))
    check_select(s, seg)


@pytest.mark.parametrize("n", [16384, 16385, 16896, 16897])
def test_select_path_boundary(n):
    """Prompts at the switch from the one-workgroup kernel (up to 16384 tokens) to the multi-workgroup path, with
    512-token slices that end exactly at the prompt's end (16896) or leave a last slice of one token (16385,
    16897); budgets at both ends and in the middle, alone and in a batch with a short prompt."""
    _say("select path boundary", n)
    for k in (1, 2048, n - 65):
        seg = W.single_segment(n - 64, 64, k)
        s = W.mixture_scores(13, seg, k_marks=(2048,))
        check_select(s, seg)
    seg = W.Segments([0, n, n + 700], [0, 0], [n - 64, 690], [2048, 100])
    s = W.mixture_scores(14, seg)
    check_select(s, seg)


def test_select_deterministic():
    _say("select determinism")
    seg = W.single_segment(32704, 64, 2048)
    s = W.mixture_scores(3, seg, k_marks=(2048,))
    a, _ = run_select(s, seg)
    b, _ = run_select(s, seg)
    assert np.array_equal(a, b)


# ----------------------------------------------------------------------------- compact


def test_compact_bit_exact():
    import torch
    _say("compact")
    tg = _tg()
    rng = np.random.default_rng(5)
    n, m = 3000, 700
    idx = np.sort(rng.choice(n, m, replace=False)).astype(np.int32)
    a = rng.integers(0, 2 ** 16, size=(n, 16, 128), dtype=np.uint16)  # 4096-byte rows
    b = rng.integers(0, 2 ** 16, size=(n, 8, 128), dtype=np.uint16)
    c = rng.standard_normal(n).astype(np.float32)  # 4-byte rows
    e = rng.integers(0, 256, size=(n, 6), dtype=np.uint8)  # 6-byte rows: byte path
    f = rng.integers(0, 2 ** 31, size=(n, 3), dtype=np.int32)  # 12-byte rows: 4-byte path
    srcs = [torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).cuda() for x in (a, b, c, e, f)]
    dsts = [torch.empty((m,) + tuple(s.shape[1:]), dtype=s.dtype, device="cuda") for s in srcs]
    tg.compact_kept(torch.from_numpy(idx).cuda(), list(zip(srcs, dsts)))
    for x, dt in zip((a, b, c, e, f), dsts):
        got = dt.cpu().numpy()
        ref = oracle.compact_rows(x, idx)
        assert got.tobytes() == ref.tobytes()


def test_compact_strided_destination():
    import torch
    _say("compact strided")
    tg = _tg()
    rng = np.random.default_rng(6)
    n, m = 1000, 333
    idx = rng.choice(n, m, replace=False).astype(np.int32)  # any order, repeats not needed
    src = torch.from_numpy(rng.standard_normal((n, 64)).astype(np.float32)).cuda()
    big = torch.zeros((m, 80), dtype=torch.float32, device="cuda")
    tg.compact_kept(torch.from_numpy(idx).cuda(), [(src, big[:, :64])])
    got = big.cpu().numpy()
    assert got[:, :64].tobytes() == oracle.compact_rows(src.cpu().numpy(), idx).tobytes()
    assert np.all(got[:, 64:] == 0)


# ----------------------------------------------------------------------------- attention


def run_attention(q, k, v, s, tau, gain, seg_offsets, use_bias=True, use_tau=True):
    tg = _tg()
    n_seg = len(seg_offsets) - 1
    lens = np.diff(seg_offsets)
    plan = tg.plan_segments(list(seg_offsets), [0] * n_seg, [0] * n_seg, [0] * n_seg, device="cuda")
    assert plan.total_kept == q.shape[0] and plan.table[:, 6].tolist() == lens.tolist()
    out = tg.gated_attention_prefill(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_f32(s) if use_bias else None,
                                     dev_f32(tau) if use_tau else None, dev_f32(gain) if use_bias else None, plan)
    return W.bf16_bits_to_f64(host_bf16(out))


def check_attention(got, q, k, v, s, tau, gain, offs, rows=None, use_bias=True, use_tau=True):
    ref = oracle.gated_attention(f64(q), f64(k), f64(v), s.astype(np.float64) if use_bias else None,
                                 tau.astype(np.float64) if use_tau else None,
                                 gain.astype(np.float64) if use_bias else None, offs, rows=rows)
    g = got if rows is None else got[rows]
    err = np.abs(g - ref).max()
    assert err <= ATTN_ATOL, f"max abs err {err:.3e}"
    return err


def compacted(L, k_budget, scores):
    seg = L.segments.with_budget(k_budget)
    idx, offs = oracle.kept_indices(scores, seg.seg_start, seg.doc_begin, seg.doc_end, seg.k_budget)
    return (oracle.compact_rows(L.q, idx), oracle.compact_rows(L.k, idx), oracle.compact_rows(L.v, idx),
            oracle.compact_rows(scores, idx).astype(np.float32), offs)


def test_attention_workload_1():
    _say("attention workload 1")
    L = layer(1)
    s = oracle_gate(L).astype(np.float32)
    q, k, v, sc, offs = compacted(L, 128, s)
    assert q.shape[0] == 192
    got = run_attention(q, k, v, sc, L.tau, L.gain, offs)
    check_attention(got, q, k, v, sc, L.tau, L.gain, offs)


@pytest.mark.parametrize("d,hq,hkv", [(64, 4, 4), (64, 4, 2), (64, 8, 2), (128, 2, 2), (128, 8, 4), (128, 8, 2)])
def test_attention_ragged_shapes(d, hq, hkv):
    _say("attention ragged", d, hq, hkv)
    rng = np.random.default_rng(d * 100 + hq * 10 + hkv)
    lens = [1, 63, 64, 65, 130, 0, 257]
    offs = np.concatenate([[0], np.cumsum(lens)])
    m = int(offs[-1])
    q = W.f32_to_bf16_bits(rng.standard_normal((m, hq, d)).astype(np.float32))
    k = W.f32_to_bf16_bits(rng.standard_normal((m, hkv, d)).astype(np.float32))
    v = W.f32_to_bf16_bits(rng.standard_normal((m, hkv, d)).astype(np.float32))
    s = rng.standard_normal(m).astype(np.float32)
    tau = rng.uniform(0.8, 1.2, hq).astype(np.float32)
    gain = rng.uniform(0.5, 1.5, hq).astype(np.float32)
    got = run_attention(q, k, v, s, tau, gain, offs)
    check_attention(got, q, k, v, s, tau, gain, offs)
    got = run_attention(q, k, v, s, tau, gain, offs, use_bias=False, use_tau=False)
    check_attention(got, q, k, v, s, tau, gain, offs, use_bias=False, use_tau=False)


def test_attention_workload_2_full():
    _say("attention workload 2 (M=2112)")
    L = layer(2)
    s = W.mixture_scores(2, L.segments)  # any fp32 score array works as the gate input
    q, k, v, sc, offs = compacted(L, 2048, s)
    assert q.shape[0] == 2112
    got = run_attention(q, k, v, sc, L.tau, L.gain, offs)
    check_attention(got, q, k, v, sc, L.tau, L.gain, offs)


@pytest.mark.parametrize("kb", [1024, 2048, 4096, 8192])
def test_attention_workload_3_sampled(kb):
    _say("attention workload 3", kb)
    L = layer(3)
    s = W.mixture_scores(3, L.segments, k_marks=(1024, 2048, 4096, 8192))
    q, k, v, sc, offs = compacted(L, kb, s)
    m = q.shape[0]
    got = run_attention(q, k, v, sc, L.tau, L.gain, offs)
    rng = np.random.default_rng(kb)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, m - 65, m - 64, m - 2, m - 1], rng.integers(0, m, 120)]))
    check_attention(got, q, k, v, sc, L.tau, L.gain, offs, rows=rows)


@pytest.mark.parametrize("d,hq,hkv,lens", [(128, 16, 8, [16384]), (64, 4, 2, [512, 3, 1000]),
                                           (128, 8, 8, [700, 65]), (128, 16, 4, [2000, 1])])
def test_attention_gather_equals_compacted(d, hq, hkv, lens):
    """Gather on load (Q/K/V/scores read through the kept indices) gives the
    compacted path's outputs bit for bit, and both match the oracle."""
    import torch
    _say("attention gather", d, hq, hkv, lens)
    tg = _tg()
    rng = np.random.default_rng(d + hq + len(lens))
    offs = np.concatenate([[0], np.cumsum(lens)])
    n = int(offs[-1])
    q = W.f32_to_bf16_bits(rng.standard_normal((n, hq, d)).astype(np.float32))
    k = W.f32_to_bf16_bits(rng.standard_normal((n, hkv, d)).astype(np.float32))
    v = W.f32_to_bf16_bits(rng.standard_normal((n, hkv, d)).astype(np.float32))
    s = rng.standard_normal(n).astype(np.float32)
    tau = rng.uniform(0.8, 1.2, hq).astype(np.float32)
    gain = rng.uniform(0.5, 1.5, hq).astype(np.float32)
    # prompts whose documents are all but the last few tokens; budgets keep about a quarter
    n_seg = len(lens)
    db = [0] * n_seg
    de = [max(0, L - 3) for L in lens]
    kb = [max(0, (L - 3) // 4) for L in lens]
    plan = tg.plan_segments(list(offs), db, de, kb, device="cuda")
    kept = tg.select_topk(dev_f32(s), plan)
    idx = kept.cpu().numpy().astype(np.int64)
    qd, kd, vd, sd = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_f32(s)
    tt, gg = dev_f32(tau), dev_f32(gain)
    got_g = tg.gated_attention_prefill_gather(qd, kd, vd, sd, tt, gg, plan, kept)
    qc, kc, vc, sc = (torch.index_select(t, 0, kept.long()) for t in (qd, kd, vd, sd))
    got_c = tg.gated_attention_prefill(qc.contiguous(), kc.contiguous(), vc.contiguous(), sc.contiguous(), tt, gg,
                                       plan)
    torch.cuda.synchronize()
    assert torch.equal(got_g.view(torch.int16), got_c.view(torch.int16))
    koffs = plan.kept_offsets
    ref_rows = np.linspace(0, idx.size - 1, min(idx.size, 300)).astype(np.int64)
    check_attention(W.bf16_bits_to_f64(host_bf16(got_g)), q[idx], k[idx], v[idx], s[idx], tau, gain, koffs,
                    rows=np.unique(ref_rows))


@pytest.mark.parametrize("d,hq,hkv", [(128, 8, 4), (64, 4, 4)])
def test_attention_gather_long_prompt(d, hq, hkv):
    """Gather on load past 8192 kept rows in a prompt (the register-staged kernel, whose row indices fill up to
    64 KiB of LDS) next to a short prompt: equal to the compacted path (direct-to-LDS kernel) bit for bit, and
    to the oracle on sampled rows."""
    import torch
    _say("attention gather long prompt", d, hq, hkv)
    tg = _tg()
    rng = np.random.default_rng(40 + d + hq)
    lens = [10000, 300]
    offs = np.concatenate([[0], np.cumsum(lens)])
    n = int(offs[-1])
    q = W.f32_to_bf16_bits(rng.standard_normal((n, hq, d)).astype(np.float32))
    k = W.f32_to_bf16_bits(rng.standard_normal((n, hkv, d)).astype(np.float32))
    v = W.f32_to_bf16_bits(rng.standard_normal((n, hkv, d)).astype(np.float32))
    s = rng.standard_normal(n).astype(np.float32)
    tau = rng.uniform(0.8, 1.2, hq).astype(np.float32)
    gain = rng.uniform(0.5, 1.5, hq).astype(np.float32)
    plan = tg.plan_segments(list(offs), [0, 0], [9990, 290], [9000, 50], device="cuda")
    assert plan.info.max_kept_len > 8192
    kept = tg.select_topk(dev_f32(s), plan)
    idx = kept.cpu().numpy().astype(np.int64)
    qd, kd, vd, sd = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_f32(s)
    tt, gg = dev_f32(tau), dev_f32(gain)
    got_g = tg.gated_attention_prefill_gather(qd, kd, vd, sd, tt, gg, plan, kept)
    qc, kc, vc, sc = (torch.index_select(t, 0, kept.long()) for t in (qd, kd, vd, sd))
    got_c = tg.gated_attention_prefill(qc.contiguous(), kc.contiguous(), vc.contiguous(), sc.contiguous(), tt, gg,
                                       plan)
    torch.cuda.synchronize()
    # the two kernels take the same products in the same order: equal bit for bit
    assert torch.equal(got_g.view(torch.int16), got_c.view(torch.int16))
    koffs = plan.kept_offsets
    ref_rows = np.unique(np.concatenate([[0, 1, 8191, 8192, 8193, 9009, 9010, idx.size - 1],
                                         np.linspace(0, idx.size - 1, 150).astype(np.int64)]))
    check_attention(W.bf16_bits_to_f64(host_bf16(got_g)), q[idx], k[idx], v[idx], s[idx], tau, gain, koffs,
                    rows=ref_rows)


def run_attention_query_tau(q, k, v, s, sigma, gain, pos, offs, use_bias=True):
    import torch
    tg = _tg()
    n_seg = len(offs) - 1
    plan = tg.plan_segments(list(offs), [0] * n_seg, [0] * n_seg, [0] * n_seg, device="cuda")
    out = tg.gated_attention_prefill_query_tau(dev_bf16(q), dev_bf16(k), dev_bf16(v),
                                               dev_f32(s) if use_bias else None, dev_f32(sigma),
                                               dev_f32(gain) if use_bias else None,
                                               torch.from_numpy(np.asarray(pos, dtype=np.int32)).cuda(), plan)
    return W.bf16_bits_to_f64(host_bf16(out))


def check_attention_query_tau(got, q, k, v, s, sigma, gain, pos, offs, rows=None, use_bias=True):
    tau = oracle.query_temperature(np.asarray(sigma, dtype=np.float64), pos, offs)
    ref = oracle.gated_attention(f64(q), f64(k), f64(v), s.astype(np.float64) if use_bias else None, tau,
                                 gain.astype(np.float64) if use_bias else None, offs, rows=rows)
    g = got if rows is None else got[rows]
    err = np.abs(g - ref).max()
    assert err <= ATTN_ATOL, f"max abs err {err:.3e}"
    return err


def kept_positions(rng, lens, keep_all=()):
    """Original positions of the kept rows of each prompt: a sorted random
    subset of a prompt about four times longer (all of it for prompts listed
    in keep_all)."""
    out = []
    for i, n in enumerate(lens):
        if i in keep_all:
            out.append(np.arange(n))
        else:
            out.append(np.sort(rng.choice(4 * n + 3, n, replace=False)))
    return np.concatenate(out).astype(np.int64) if out else np.zeros(0, np.int64)


@pytest.mark.parametrize("d,hq,hkv", [(64, 4, 2), (64, 8, 2), (128, 2, 2), (128, 16, 8), (128, 16, 4)])
def test_attention_query_tau_ragged(d, hq, hkv):
    _say("attention query tau ragged", d, hq, hkv)
    rng = np.random.default_rng(d + 7 * hq + hkv)
    lens = [1, 63, 64, 65, 130, 0, 257]
    offs = np.concatenate([[0], np.cumsum(lens)])
    m = int(offs[-1])
    q = W.f32_to_bf16_bits(rng.standard_normal((m, hq, d)).astype(np.float32))
    k = W.f32_to_bf16_bits(rng.standard_normal((m, hkv, d)).astype(np.float32))
    v = W.f32_to_bf16_bits(rng.standard_normal((m, hkv, d)).astype(np.float32))
    s = rng.standard_normal(m).astype(np.float32)
    sigma = rng.uniform(-1.0, 1.5, hq).astype(np.float32)
    sigma[0] = -40.0  # softplus ~ 4e-18: the bias alone
    if hq > 2:
        sigma[1] = 25.0  # the large-sigma branch of softplus
    gain = rng.uniform(0.5, 1.5, hq).astype(np.float32)
    pos = kept_positions(rng, lens, keep_all=(4,))
    got = run_attention_query_tau(q, k, v, s, sigma, gain, pos, offs)
    check_attention_query_tau(got, q, k, v, s, sigma, gain, pos, offs)
    got = run_attention_query_tau(q, k, v, s, sigma, gain, pos, offs, use_bias=False)
    check_attention_query_tau(got, q, k, v, s, sigma, gain, pos, offs, use_bias=False)


@pytest.mark.parametrize("idx,kb", [(2, 2048), (3, 8192)])
def test_attention_query_tau_workloads(idx, kb):
    """The kept rows of workloads 2 and 3 with their true original positions;
    every row of workload 2 (M = 2112), sampled rows of workload 3 (M = 8256)."""
    _say("attention query tau workload", idx, kb)
    L = layer(idx)
    s = W.mixture_scores(idx, L.segments, k_marks=(1024, 2048, 4096, 8192))
    seg = L.segments.with_budget(kb)
    kept, offs = oracle.kept_indices(s, seg.seg_start, seg.doc_begin, seg.doc_end, seg.k_budget)
    starts = np.repeat(np.asarray(seg.seg_start[:-1]), np.diff(offs))
    pos = kept - starts
    q, k, v = (oracle.compact_rows(t, kept) for t in (L.q, L.k, L.v))
    sc = oracle.compact_rows(s, kept).astype(np.float32)
    m = q.shape[0]
    rng = np.random.default_rng(kb)
    sigma = rng.uniform(-0.5, 1.0, L.tau.size).astype(np.float32)
    got = run_attention_query_tau(q, k, v, sc, sigma, L.gain, pos, offs)
    rows = None
    if m > 4000:
        rows = np.unique(np.concatenate([[0, 1, 63, 64, m - 65, m - 64, m - 2, m - 1], rng.integers(0, m, 120)]))
    check_attention_query_tau(got, q, k, v, sc, sigma, L.gain, pos, offs, rows=rows)


def test_attention_deterministic():
    _say("attention determinism")
    L = layer(1)
    s = oracle_gate(L).astype(np.float32)
    q, k, v, sc, offs = compacted(L, 128, s)
    a = run_attention(q, k, v, sc, L.tau, L.gain, offs)
    b = run_attention(q, k, v, sc, L.tau, L.gain, offs)
    assert a.tobytes() == b.tobytes()


# ----------------------------------------------------------------------------- pipeline


@pytest.mark.parametrize("idx", [1, 2])
def test_pipeline(idx):
    """gate -> select -> compact -> attention on the GPU, each stage against the oracle."""
    import torch
    _say("pipeline workload", idx)
    tg = _tg()
    L = layer(idx)
    seg = L.segments
    plan = tg.plan_from(seg, device="cuda")
    x, qd, kd, vd = dev_bf16(L.x), dev_bf16(L.q), dev_bf16(L.k), dev_bf16(L.v)
    s_gpu = tg.gate_score(x, dev_bf16(L.w1), None, dev_f32(L.w2), 0.0, plan)
    idx_gpu = tg.select_topk(s_gpu, plan)
    m = plan.total_kept
    hc = torch.empty((m, L.d), dtype=torch.bfloat16, device="cuda")
    qc = torch.empty((m, L.hq, L.head_dim), dtype=torch.bfloat16, device="cuda")
    kc = torch.empty((m, L.hkv, L.head_dim), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    sc = torch.empty(m, dtype=torch.float32, device="cuda")
    tg.compact_kept(idx_gpu, [(x, hc), (qd, qc), (kd, kc), (vd, vc), (s_gpu, sc)])
    o = tg.gated_attention_prefill(qc, kc, vc, sc, dev_f32(L.tau), dev_f32(L.gain), plan)
    torch.cuda.synchronize()

    s_ref = oracle_gate(L)
    s_got = s_gpu.cpu().numpy()
    check_scores(s_got, s_ref, doc_mask_of(seg))
    ref_idx, offs = oracle.kept_indices(s_ref, seg.seg_start, seg.doc_begin, seg.doc_end, seg.k_budget)
    got_idx = idx_gpu.cpu().numpy().astype(np.int64)
    # the select is exact on the fp32 scores the gate wrote
    own_idx, _ = oracle.kept_indices(s_got.astype(np.float64), seg.seg_start, seg.doc_begin, seg.doc_end,
                                     seg.k_budget)
    assert np.array_equal(got_idx, own_idx), "select differs from the oracle on the GPU's own scores"
    assert got_idx.size == ref_idx.size
    if not np.array_equal(got_idx, ref_idx):
        # allowed only at near-ties of the oracle scores (GPU and oracle scores differ by rounding); the later
        # stages are then checked on the GPU's kept set
        sym = np.setxor1d(got_idx, ref_idx)
        t = np.sort(s_ref[seg.doc_begin[0]:seg.doc_end[0]])[::-1][seg.k_budget[0] - 1]
        assert np.all(np.abs(s_ref[sym] - t) <= 4 * SCORE_RTOL * max(1.0, abs(t))), "kept sets differ beyond near-ties"
        _say("kept sets differ at a near-tie:", sym.size, "tokens; checking the later stages on the GPU's set")
    assert hc.view(torch.int16).cpu().numpy().tobytes() == oracle.compact_rows(L.x.view(np.int16), got_idx).tobytes()
    got = W.bf16_bits_to_f64(host_bf16(o))
    q, k, v = (oracle.compact_rows(a, got_idx) for a in (L.q, L.k, L.v))
    # the oracle's own scores drive its attention: gate error feeds through the bias (|g| <= 1.5)
    check_attention(got, q, k, v, oracle.compact_rows(s_ref, got_idx), L.tau, L.gain, offs)


@pytest.mark.parametrize("kb", [2048, 4096])
def test_pipeline_workload_4_graph(kb):
    """The long-context layer at full size (131008 documents + 64 question tokens, d = 2048, 16 Q / 8 KV heads)
    run as bench.py times it: the whole step captured as one HIP graph and replayed.  Gate scores against the
    oracle per element; the kept set exactly the oracle's on the GPU's own scores (and the oracle's scores'
    set up to near-ties); the compacted hidden rows bit for bit; the attention against the oracle on sampled
    rows of the M = kb + 64 kept rows."""
    import torch
    import bench
    _say("pipeline workload 4 graph", kb)
    tg = _tg()
    L = layer(4)
    pipe = bench.Pipeline(L, kb, torch, tg)
    g = bench.capture_step(pipe)
    for t in (pipe.scores, pipe.out, pipe.hc):
        t.zero_()
    pipe.kept.fill_(-1)
    g.replay()
    torch.cuda.synchronize()
    seg = pipe.seg
    s_got = pipe.scores.cpu().numpy()
    got_idx = pipe.kept.cpu().numpy().astype(np.int64)
    s_ref = oracle_gate(L)
    check_scores(s_got, s_ref, doc_mask_of(seg))
    own_idx, offs = oracle.kept_indices(s_got.astype(np.float64), seg.seg_start, seg.doc_begin, seg.doc_end,
                                        seg.k_budget)
    assert np.array_equal(got_idx, own_idx), "select differs from the oracle on the GPU's own scores"
    ref_idx, _ = oracle.kept_indices(s_ref, seg.seg_start, seg.doc_begin, seg.doc_end, seg.k_budget)
    if not np.array_equal(got_idx, ref_idx):
        sym = np.setxor1d(got_idx, ref_idx)
        t = np.sort(s_ref[seg.doc_begin[0]:seg.doc_end[0]])[::-1][seg.k_budget[0] - 1]
        assert np.all(np.abs(s_ref[sym] - t) <= 4 * SCORE_RTOL * max(1.0, abs(t))), "kept sets differ beyond near-ties"
        _say("kept sets differ at a near-tie:", sym.size, "tokens")
    assert pipe.hc.view(torch.int16).cpu().numpy().tobytes() == oracle.compact_rows(L.x.view(np.int16), got_idx).tobytes()
    m = got_idx.size
    assert m == kb + 64
    rng = np.random.default_rng(kb)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, m // 2, m - 65, m - 64, m - 2, m - 1], rng.integers(0, m, 60)]))
    got = W.bf16_bits_to_f64(host_bf16(pipe.out))
    q, k, v = (oracle.compact_rows(a, got_idx) for a in (L.q, L.k, L.v))
    check_attention(got, q, k, v, oracle.compact_rows(s_ref, got_idx), L.tau, L.gain, offs, rows=rows)


@pytest.mark.parametrize("gather", [False, True])
def test_pipeline_graph_replays_match_eager(gather):
    """The step captured as a HIP graph (as bench.py times it): every replay,
    with eager launches and synchronisations in between, gives the eager
    results bit for bit."""
    _say("pipeline graph replay")
    import torch
    import bench
    tg = _tg()
    L = layer(1)
    pipe = bench.Pipeline(L, 128, torch, tg, gather=gather)
    for _, f in pipe.stages():
        f()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (pipe.scores, pipe.kept, pipe.out, pipe.hc)]
    g = bench.capture_step(pipe)
    for rep in range(4):
        for t in (pipe.scores, pipe.out, pipe.hc):
            t.zero_()
        pipe.kept.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        got = (pipe.scores, pipe.kept, pipe.out, pipe.hc)
        for a, b in zip(got, ref):
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.int32 else a,
                               b.view(torch.uint8) if b.dtype != torch.int32 else b), f"replay {rep}"
        for _, f in pipe.stages():  # eager work between replays
            f()
        torch.cuda.synchronize()
