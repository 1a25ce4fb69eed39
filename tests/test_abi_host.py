"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, and rejects bad arguments before touching any device (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from _lib import ROOT, binding, gpu_available

tg = binding()
L = tg._lib
FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(os.path.join(ROOT, "include", "tokengate.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tg_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n
    assert set(tg.EXPORTS) <= set(names)
    assert tg.abi_version() == 1
    assert tg.status_string(0) == "ok" and tg.status_string(-3).startswith("workspace")


def test_single_hip_runtime_in_process():
    import torch  # noqa: F401
    assert len(tg.hip_runtimes_loaded()) <= 1


def test_plan_segments_matches_oracle_counts():
    rng = np.random.default_rng(0)
    from learned_token_pruning_amd import workloads
    seg = workloads.random_segments(rng, 20, 50)
    p = tg.plan_from(seg)
    assert p.n_tokens == seg.n_tokens
    expect = [oracle.kept_count(seg.n_doc(i), seg.seg_len(i) - seg.n_doc(i), seg.k_budget[i]) for i in range(seg.n_seg)]
    assert p.table[:, 6].tolist() == expect
    assert p.total_kept == sum(expect)
    assert p.kept_offsets.tolist() == np.concatenate([[0], np.cumsum(expect)]).tolist()
    assert p.table[:, 4].tolist() == [min(seg.k_budget[i], seg.n_doc(i)) for i in range(seg.n_seg)]
    assert p.info.max_seg_len == max(seg.seg_len(i) for i in range(seg.n_seg))


def test_kept_count_matches_oracle_and_plan():
    rng = np.random.default_rng(4)
    for _ in range(200):
        n_doc, n_other, k = (int(v) for v in rng.integers(0, 5000, 3))
        assert tg.kept_count(n_doc, n_other, k) == oracle.kept_count(n_doc, n_other, k)
    assert tg.kept_count(10, 3, 0) == 3 and tg.kept_count(10, 3, 99) == 13
    assert tg.kept_count(-1, 0, 0) == -1 and tg.kept_count(0, -1, 0) == -1 and tg.kept_count(5, 0, -1) == -1
    p = tg.plan_segments([0, 100, 164], [10, 0], [90, 60], [20, 500])
    assert p.table[:, 6].tolist() == [tg.kept_count(80, 20, 20), tg.kept_count(60, 4, 500)]


@pytest.mark.parametrize("args", [
    ([0, 5], [0], [5], [-1]),       # negative budget
    ([0, 5], [0], [6], [1]),        # span past the prompt
    ([0, 5], [3], [2], [1]),        # reversed span
    ([1, 5], [0], [2], [1]),        # seg_start[0] != 0
    ([0, 5, 4], [0, 0], [1, 0], [1, 1]),  # decreasing offsets
])
def test_plan_segments_rejects(args):
    with pytest.raises(tg.TokenGateError) as e:
        tg.plan_segments(*args)
    assert e.value.status == -1


def _plan():
    return tg.plan_segments([0, 100], [0], [90], [10])


def test_gate_validation():
    p = _plan()
    info = ctypes.byref(p.info)
    f = L.tg_gate_score
    ws = tg.gate_workspace_bytes(p, 2048, 256)
    assert ws >= 8 and ws % 256 == 0
    # null x
    assert f(None, 2048, 2048, FAKE, None, FAKE, 0.0, 256, FAKE, info, 1e-6, FAKE, FAKE, ws, None) == -1
    # d not a multiple of 64, h too large, misaligned ld
    assert f(FAKE, 2048, 2040, FAKE, None, FAKE, 0.0, 256, FAKE, info, 1e-6, FAKE, FAKE, ws, None) == -2
    assert f(FAKE, 2048, 2048, FAKE, None, FAKE, 0.0, 320, FAKE, info, 1e-6, FAKE, FAKE, ws, None) == -2
    assert f(FAKE, 2052, 2048, FAKE, None, FAKE, 0.0, 256, FAKE, info, 1e-6, FAKE, FAKE, ws, None) == -2
    # ld_x < d
    assert f(FAKE, 1024, 2048, FAKE, None, FAKE, 0.0, 256, FAKE, info, 1e-6, FAKE, FAKE, ws, None) == -1
    # NaN eps
    assert f(FAKE, 2048, 2048, FAKE, None, FAKE, 0.0, 256, FAKE, info, float("nan"), FAKE, FAKE, ws, None) == -1
    # workspace too small / misaligned
    assert f(FAKE, 2048, 2048, FAKE, None, FAKE, 0.0, 256, FAKE, info, 1e-6, FAKE, FAKE, ws - 1, None) == -3
    assert f(FAKE, 2048, 2048, FAKE, None, FAKE, 0.0, 256, FAKE, info, 1e-6, FAKE, ctypes.c_void_p(0x10010), ws,
             None) == -3
    # null segment table
    assert f(FAKE, 2048, 2048, FAKE, None, FAKE, 0.0, 256, None, info, 1e-6, FAKE, FAKE, ws, None) == -1


def test_gate_prepacked_validation():
    p = _plan()
    info = ctypes.byref(p.info)
    assert tg.gate_workspace_bytes(p, 2048, 256) > 0 and L.tg_gate_packed_w1_bytes(2048, 256) == 2048 * 256 * 2
    assert L.tg_gate_packed_w1_bytes(0, 256) == 0
    assert L.tg_gate_pack_w1(None, 2048, 256, FAKE, None) == -1
    assert L.tg_gate_pack_w1(FAKE, 2048, 96, FAKE, None) == -2
    assert L.tg_gate_pack_w1(FAKE, 2050, 256, FAKE, None) == -2
    ws = tg.gate_workspace_bytes(p, 2048, 256)
    f = L.tg_gate_score_prepacked
    assert f(FAKE, 2048, 2048, None, None, FAKE, 0.0, 256, FAKE, info, 1e-6, FAKE, FAKE, ws, None) == -1
    assert f(FAKE, 2048, 2048, FAKE, None, FAKE, 0.0, 320, FAKE, info, 1e-6, FAKE, FAKE, ws, None) == -2
    assert f(FAKE, 2048, 2048, FAKE, None, FAKE, 0.0, 256, FAKE, info, 1e-6, FAKE, FAKE, ws - 1, None) == -3


def test_select_validation():
    p = _plan()
    info = ctypes.byref(p.info)
    ws = tg.select_workspace_bytes(p)
    assert ws >= 0
    f = L.tg_select_topk
    assert f(None, FAKE, info, FAKE, FAKE, ws, None) == -1
    assert f(FAKE, FAKE, info, None, FAKE, ws, None) == -1
    if ws > 0:
        assert f(FAKE, FAKE, info, FAKE, FAKE, ws - 4, None) == -3
        assert f(FAKE, FAKE, info, FAKE, None, ws, None) == -3
    # prompts past 16384 tokens take the multi-workgroup path, which needs a workspace
    assert ws == 0
    long = tg.plan_segments([0, 40000, 40100], [0, 0], [39000, 90], [4096, 10])  # 10 slices of 4096
    wl = tg.select_workspace_bytes(long)
    assert wl >= 4 * (3 * 2 * 2048 + 2 * 10 * 2) and wl % 256 == 0
    il = ctypes.byref(long.info)
    assert f(FAKE, FAKE, il, FAKE, None, wl, None) == -3
    assert f(FAKE, FAKE, il, FAKE, FAKE, wl - 256, None) == -3
    bad = tg.PlanInfo(n_tokens=10, total_kept=20, n_seg=1, max_seg_len=10, max_doc_len=5, max_kept_len=10)
    assert f(FAKE, FAKE, ctypes.byref(bad), FAKE, FAKE, ws, None) == -1


def test_compact_validation():
    f = L.tg_compact_kept
    V = ctypes.c_void_p
    I = ctypes.c_int64

    def arr(t, *v):
        return (t * len(v))(*v)

    src, dst = arr(V, 0x10000), arr(V, 0x20000)
    assert f(FAKE, 10, 100, 0, src, dst, arr(I, 16), arr(I, 16), arr(I, 16), None) == -1
    assert f(FAKE, 10, 100, 9, src, dst, arr(I, 16), arr(I, 16), arr(I, 16), None) == -1
    assert f(FAKE, -1, 100, 1, src, dst, arr(I, 16), arr(I, 16), arr(I, 16), None) == -1
    assert f(FAKE, 10, 100, 1, src, dst, arr(I, 32), arr(I, 32), arr(I, 16), None) == -1  # dst stride < row
    assert f(FAKE, 10, 100, 1, src, src, arr(I, 16), arr(I, 16), arr(I, 16), None) == -1  # in place
    assert f(FAKE, 10, -1, 1, src, dst, arr(I, 16), arr(I, 16), arr(I, 16), None) == -1
    assert f(None, 10, 100, 1, src, dst, arr(I, 16), arr(I, 16), arr(I, 16), None) == -1
    assert f(None, 0, 100, 1, src, dst, arr(I, 16), arr(I, 16), arr(I, 16), None) == 0  # nothing to do


def test_attention_validation():
    p = _plan()
    info = ctypes.byref(p.info)
    f = L.tg_gated_attention_prefill
    assert f(FAKE, FAKE, FAKE, None, None, None, FAKE, info, 16, 6, 128, FAKE, None) == -2  # hq % hkv
    assert f(FAKE, FAKE, FAKE, None, None, None, FAKE, info, 16, 2, 128, FAKE, None) == -2  # group 8
    assert f(FAKE, FAKE, FAKE, None, None, None, FAKE, info, 16, 8, 96, FAKE, None) == -2   # head_dim
    assert f(None, FAKE, FAKE, None, None, None, FAKE, info, 16, 8, 128, FAKE, None) == -1
    assert f(ctypes.c_void_p(0x10008), FAKE, FAKE, None, None, None, FAKE, info, 16, 8, 128, FAKE, None) == -1
    assert f(FAKE, FAKE, FAKE, None, None, None, FAKE, info, 0, 8, 128, FAKE, None) == -1


def test_attention_split_workspace():
    """Workspace of the split-tile attention: sized only for a single prompt too short to fill the GPU (the
    device's CU count, 256 on MI355X and when no device is present), zero for batches and for prompts long enough
    to fill it; the entry point validates shapes and arguments like the plain one."""
    def nbytes(lens, hq=16, hkv=8, d=128):
        p = tg.plan_segments([0] + list(np.cumsum(lens)), [0] * len(lens), [0] * len(lens), [0] * len(lens))
        return tg.attention_prefill_workspace_bytes(p, hq, hkv, d)
    if not gpu_available():
        rec = 2 * 4 * (32 * 128 + 64) * 4  # two records of 4 waves x (O^T, m, l) per split tile
        b = nbytes([2112])
        # a 256-byte header (status word), the merge counters padded to 256 bytes, then the records
        assert b > 0 and (b - 256 - 256 * ((b // rec * 8 + 255) // 256)) % rec == 0
        assert nbytes([1000]) > 0
    assert nbytes([300, 700]) == 0 and nbytes([64]) == 0 and nbytes([8192]) == 0
    assert nbytes([2112], hq=16, hkv=6) == 0 and L.tg_attention_prefill_workspace_bytes(None, 16, 8, 128) == 0
    # the status query validates before touching the device
    word = ctypes.c_int(0)
    assert L.tg_attention_workspace_status(None, ctypes.byref(word), None) == -1
    assert L.tg_attention_workspace_status(FAKE, None, None) == -1
    p = _plan()
    info = ctypes.byref(p.info)
    f = L.tg_gated_attention_prefill_ws
    assert f(FAKE, FAKE, FAKE, None, None, None, FAKE, info, 16, 6, 128, FAKE, None, 0, None) == -2
    assert f(None, FAKE, FAKE, None, None, None, FAKE, info, 16, 8, 128, FAKE, None, 0, None) == -1
    empty = tg.plan_segments([0, 0], [0], [0], [0])
    assert f(None, None, None, None, None, None, FAKE, ctypes.byref(empty.info), 16, 8, 128, None, None, 0, None) == 0


def test_attention_rejects_prompts_past_32bit_ranges():
    # 2^21 kept rows x 8 KV heads x 128 dims x 2 bytes = 2^32 bytes of K per prompt
    big = tg.plan_segments([0, 1 << 21], [0], [0], [0])
    info = ctypes.byref(big.info)
    assert L.tg_gated_attention_prefill(FAKE, FAKE, FAKE, None, None, None, FAKE, info, 16, 8, 128, FAKE, None) == -2
    assert L.tg_gated_attention_prefill_query_tau(FAKE, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, info, 16, 8, 128,
                                                  FAKE, None) == -2
    assert L.tg_gated_attention_prefill_lse(FAKE, FAKE, FAKE, None, None, None, FAKE, info, 16, 8, 128, FAKE, FAKE,
                                            None) == -2


def test_attention_gather_validation():
    p = _plan()
    info = ctypes.byref(p.info)
    f = L.tg_gated_attention_prefill_gather
    assert f(FAKE, FAKE, FAKE, None, None, None, FAKE, info, 16, 8, 128, None, 100, FAKE, None) == -1  # no indices
    assert f(FAKE, FAKE, FAKE, None, None, None, FAKE, info, 16, 8, 128, FAKE, 0, FAKE, None) == -1  # no rows
    assert f(FAKE, FAKE, FAKE, None, None, None, FAKE, info, 16, 8, 96, FAKE, 100, FAKE, None) == -2
    assert f(FAKE, FAKE, FAKE, None, None, None, FAKE, info, 16, 8, 128, FAKE, 1 << 22, FAKE, None) == -2  # 32-bit offsets
    big = tg.plan_segments([0, 40000], [0], [39000], [20000])  # more kept rows than the gather path holds
    assert f(FAKE, FAKE, FAKE, None, None, None, FAKE, ctypes.byref(big.info), 16, 8, 128, FAKE, 40000, FAKE,
             None) == -2


def test_attention_query_tau_validation():
    p = _plan()
    info = ctypes.byref(p.info)
    f = L.tg_gated_attention_prefill_query_tau
    assert f(FAKE, FAKE, FAKE, None, None, None, FAKE, FAKE, info, 16, 8, 128, FAKE, None) == -1  # no sigma
    assert f(FAKE, FAKE, FAKE, None, FAKE, None, None, FAKE, info, 16, 8, 128, FAKE, None) == -1  # no positions
    assert f(FAKE, FAKE, FAKE, None, FAKE, None, ctypes.c_void_p(0x10002), FAKE, info, 16, 8, 128, FAKE,
             None) == -1  # misaligned positions
    assert f(FAKE, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, info, 16, 8, 96, FAKE, None) == -2
    assert f(FAKE, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, info, 16, 2, 128, FAKE, None) == -2
    empty = tg.plan_segments([0, 0], [0], [0], [0])
    assert f(None, None, None, None, FAKE, None, None, FAKE, ctypes.byref(empty.info), 16, 8, 128, None, None) == 0


def test_decode_validation():
    f = L.tg_gated_attention_decode
    ws = tg.decode_workspace_bytes(2, 16, 128, 1000)
    assert ws == 2 * 16 * 4 * 130 * 4  # 4 chunks of 256 rows, D + 2 floats per head and chunk
    assert tg.decode_workspace_bytes(0, 16, 128, 10) == 0
    args = lambda **kw: dict(dict(q=FAKE, k=FAKE, v=FAKE, s=None, tau=None, tpq=0, gain=None, lens=FAKE, b=2, cap=1000,
                                  hq=16, hkv=8, d=128, out=FAKE, ws=FAKE, wsb=ws), **kw)
    call = lambda a: f(a["q"], a["k"], a["v"], a["s"], a["tau"], a["tpq"], a["gain"], a["lens"], a["b"], a["cap"],
                       a["hq"], a["hkv"], a["d"], a["out"], a["ws"], a["wsb"], None)
    assert call(args(b=0, q=None, lens=None)) == 0  # nothing to do
    assert call(args(lens=None)) == -1
    assert call(args(k=None)) == -1
    assert call(args(tpq=2)) == -1
    assert call(args(cap=-1)) == -1
    assert call(args(q=ctypes.c_void_p(0x10008))) == -1
    assert call(args(hkv=6)) == -2
    assert call(args(hkv=2)) == -2   # group of 8
    assert call(args(d=96)) == -2
    assert call(args(b=70000, wsb=1 << 40)) == -2
    assert call(args(cap=65535 * 256 + 1, wsb=1 << 40)) == -2
    assert call(args(wsb=ws - 1)) == -3
    assert call(args(ws=None)) == -3


def test_backward_validation():
    p = _plan()
    info = ctypes.byref(p.info)
    ws = tg.attention_backward_workspace_bytes(p, 16, 8, 128)
    assert ws >= (10 * 16 + 10 * 8) * 4
    f = L.tg_gated_attention_backward
    call = lambda **kw: f(*[kw.get(n, FAKE) for n in ("q", "k", "v")], None, None, None, FAKE, info, 16,
                          kw.get("hkv", 8), kw.get("d", 128), *[kw.get(n, FAKE) for n in ("out", "dout", "lse", "dq",
                                                                                           "dk", "dv")],
                          None, None, None, kw.get("ws", FAKE), kw.get("wsb", ws), None)
    assert call(dout=None) == -1
    assert call(lse=None) == -1
    assert call(dq=ctypes.c_void_p(0x10004)) == -1
    assert call(hkv=6) == -2
    assert call(d=96) == -2
    assert call(wsb=ws - 4) == -3
    assert call(ws=None) == -3
    g = L.tg_gated_attention_prefill_lse
    assert g(FAKE, FAKE, FAKE, None, None, None, FAKE, info, 16, 8, 128, FAKE, None, None) == -1  # no lse
    assert g(FAKE, FAKE, FAKE, None, None, None, FAKE, info, 16, 8, 96, FAKE, FAKE, None) == -2


@pytest.mark.skipif(gpu_available(), reason="only meaningful without a GPU: valid calls must report no device")
def test_valid_calls_report_no_device_without_gpu():
    p = _plan()
    info = ctypes.byref(p.info)
    ws = tg.gate_workspace_bytes(p, 2048, 256)
    assert L.tg_gate_score(FAKE, 2048, 2048, FAKE, None, FAKE, 0.0, 256, FAKE, info, 1e-6, FAKE, FAKE, ws, None) == -4
    assert L.tg_select_topk(FAKE, FAKE, info, FAKE, FAKE, tg.select_workspace_bytes(p), None) == -4
    assert L.tg_gate_pack_w1(FAKE, 2048, 256, FAKE, None) == -4
    assert L.tg_gate_score_prepacked(FAKE, 2048, 2048, FAKE, None, FAKE, 0.0, 256, FAKE, info, 1e-6, FAKE, FAKE, ws,
                                     None) == -4
    assert L.tg_gated_attention_prefill(FAKE, FAKE, FAKE, None, None, None, FAKE, info, 16, 8, 128, FAKE, None) == -4
    assert L.tg_gated_attention_prefill_query_tau(FAKE, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, info, 16, 8, 128,
                                                  FAKE, None) == -4
    assert L.tg_gated_attention_decode(FAKE, FAKE, FAKE, None, None, 0, None, FAKE, 2, 1000, 16, 8, 128, FAKE, FAKE,
                                       tg.decode_workspace_bytes(2, 16, 128, 1000), None) == -4
    assert L.tg_gated_attention_prefill_lse(FAKE, FAKE, FAKE, None, None, None, FAKE, info, 16, 8, 128, FAKE, FAKE,
                                            None) == -4
    assert L.tg_gated_attention_backward(FAKE, FAKE, FAKE, None, None, None, FAKE, info, 16, 8, 128, FAKE, FAKE, FAKE,
                                         FAKE, FAKE, FAKE, None, None, None, FAKE,
                                         tg.attention_backward_workspace_bytes(p, 16, 8, 128), None) == -4


def test_dense_validation():
    V = ctypes.c_void_p
    g = L.tg_gemm_bf16
    # bad epilogue, n not a multiple of 128, k not a multiple of 64, ld too small, missing residual
    assert g(3, FAKE, 256, FAKE, 256, 10, 128, 256, None, 0, FAKE, 128, None) == -1
    assert g(0, FAKE, 256, FAKE, 256, 10, 100, 256, None, 0, FAKE, 128, None) == -2
    assert g(0, FAKE, 256, FAKE, 256, 10, 128, 200, None, 0, FAKE, 128, None) == -2
    assert g(0, FAKE, 100, FAKE, 256, 10, 128, 256, None, 0, FAKE, 128, None) == -1
    assert g(1, FAKE, 256, FAKE, 256, 10, 128, 256, None, 0, FAKE, 128, None) == -1
    assert g(0, None, 256, None, 256, 0, 128, 256, None, 0, None, 128, None) == 0  # empty
    r = L.tg_rmsnorm_bf16
    assert r(FAKE, 256, 10, 250, FAKE, 1e-6, FAKE, 256, None) == -2
    assert r(FAKE, 256, 10, 256, FAKE, -1.0, FAKE, 256, None) == -1
    rp = L.tg_rope_split_bf16
    assert rp(FAKE, 4096, 10, 16, 8, 128, FAKE, 0.5, FAKE, FAKE, FAKE, None) == -1  # theta <= 1
    assert rp(FAKE, 1000, 10, 16, 8, 128, FAKE, 1e6, FAKE, FAKE, FAKE, None) == -1  # ld too small
    p = _plan()
    info = ctypes.byref(p.info)
    w = tg.LayerWeights(0x10000, 0x10000, 0x10000, 0x10000, 0x10000, 0x10000, None, None)
    ws = tg.decoder_layer_workspace_bytes(p.total_kept, 2048, 16, 8, 128, 6144)
    assert ws > 0
    dl = L.tg_decoder_layer
    assert dl(FAKE, FAKE, None, FAKE, info, 2048, 16, 8, 96, 6144, 1e-6, 1e6, ctypes.byref(w), None, FAKE, ws,
              None) == -2  # head_dim
    assert dl(FAKE, FAKE, None, FAKE, info, 2048, 16, 8, 128, 6144, 1e-6, 1e6, ctypes.byref(w), None, FAKE, ws - 1,
              None) == -3
    assert dl(FAKE, FAKE, None, FAKE, info, 2048, 16, 8, 128, 6144, 1e-6, 1e6, None, None, FAKE, ws, None) == -1
