"""Pins of the oracle's dense decoder stack: the bf16 format definition,
closed forms and invariances of RMSNorm / RoPE / SiLU, a layer against the
same layer assembled from torch library routines (float64), the pruned
stack reducing to the unpruned stack when nothing is pruned, and the pruned
stack's kept rows equal to a full-length forward that keeps every token at
its original position and masks the pruned keys out of the attention above
the gate (with and without the gate bias)."""
import math

import numpy as np
import pytest
import torch

import oracle


def test_round_bf16_definition():
    v = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -7, -2.5, 3.0e38, 1e-40, 0.0])
    got = oracle.round_bf16(v)
    # halfway cases go to the even significand; 1 + 2^-7 is exactly representable
    exp = np.array([1.0, 1.0, 1 + 4 * 2 ** -8, 1 + 2 ** -7, -2.5, got[5], got[6], 0.0])
    np.testing.assert_array_equal(got[[0, 1, 2, 3, 4, 7]], exp[[0, 1, 2, 3, 4, 7]])
    assert abs(got[5] - 3.0e38) / 3.0e38 <= 2 ** -8
    x = np.random.default_rng(0).standard_normal(5000)
    r = oracle.round_bf16(x)
    assert np.all(np.abs(r - x) <= 2 ** -8 * np.abs(x))
    assert np.array_equal(oracle.round_bf16(r), r)  # idempotent


def test_rmsnorm_closed_forms():
    w = np.array([1.0, 2.0, -1.0, 0.5])
    x = np.full((1, 4), -3.0)
    np.testing.assert_allclose(oracle.rmsnorm(x, w, 0.0), -w[None, :], rtol=1e-15)
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 64))
    np.testing.assert_allclose(oracle.rmsnorm(7.0 * x, np.ones(64), 0.0), oracle.rmsnorm(x, np.ones(64), 0.0),
                               rtol=1e-13)
    y = oracle.rmsnorm(x, np.ones(64), 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-13)


def test_rope_rotation_properties():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((6, 3, 16))
    k = rng.standard_normal((6, 3, 16))
    pos = np.array([0, 1, 5, 100, 4095, 65535])
    qr = oracle.rope(q, pos, 1e6)
    np.testing.assert_allclose(qr[0], q[0], rtol=0, atol=0)  # position 0 is the identity
    # each pair (i, i + D/2) keeps its length
    half = 8
    np.testing.assert_allclose(qr[..., :half] ** 2 + qr[..., half:] ** 2, q[..., :half] ** 2 + q[..., half:] ** 2,
                               rtol=1e-12)
    # q(p) . k(p') depends only on p - p'
    a = np.einsum("hd,hd->h", oracle.rope(q[1:2], [7], 1e4)[0], oracle.rope(k[2:3], [3], 1e4)[0])
    b = np.einsum("hd,hd->h", oracle.rope(q[1:2], [1007], 1e4)[0], oracle.rope(k[2:3], [1003], 1e4)[0])
    np.testing.assert_allclose(a, b, rtol=1e-9)
    # the first pair rotates by exactly p radians
    e = np.zeros((1, 1, 16)); e[0, 0, 0] = 1.0
    np.testing.assert_allclose(oracle.rope(e, [2], 1e6)[0, 0, [0, 8]], [math.cos(2), math.sin(2)], rtol=1e-15)


def test_silu_antisymmetry():
    x = np.linspace(-20, 20, 101)
    np.testing.assert_allclose(oracle.silu(x) - oracle.silu(-x), x, rtol=1e-13, atol=1e-13)


def _layer(rng, d, hq, hkv, dh, f, gated=False):
    s = 0.02
    mk = lambda *shape: rng.standard_normal(shape) * s
    tau = rng.uniform(0.8, 1.2, hq) if gated else None
    gain = rng.uniform(0.5, 1.5, hq) if gated else None
    return oracle.LayerWeights(1.0 + 0.1 * rng.standard_normal(d), mk(hq * dh, d), mk(hkv * dh, d), mk(hkv * dh, d),
                               mk(d, hq * dh), 1.0 + 0.1 * rng.standard_normal(d), mk(f, d), mk(f, d), mk(d, f),
                               tau, gain)


def _torch_layer(x, pos, w, hq, hkv, dh, eps, theta):
    """The same layer from torch library routines in float64 (causal, no gate)."""
    F = torch.nn.functional
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    X = t(x)
    m, d = X.shape
    xn = F.rms_norm(X, (d,), t(w.attn_norm), eps)
    q = (xn @ t(w.wq).T).reshape(m, hq, dh)
    k = (xn @ t(w.wk).T).reshape(m, hkv, dh)
    v = (xn @ t(w.wv).T).reshape(m, hkv, dh)
    half = dh // 2
    inv = theta ** (-torch.arange(half, dtype=torch.float64) * 2 / dh)
    ang = t(pos)[:, None] * inv[None, :]
    cos = torch.cat([ang.cos(), ang.cos()], -1)[:, None, :]
    sin = torch.cat([ang.sin(), ang.sin()], -1)[:, None, :]
    rot = lambda z: torch.cat([-z[..., half:], z[..., :half]], -1)
    q = q * cos + rot(q) * sin
    k = k * cos + rot(k) * sin
    rep = hq // hkv
    a = F.scaled_dot_product_attention(q.permute(1, 0, 2), k.repeat_interleave(rep, 1).permute(1, 0, 2).contiguous(),
                                       v.repeat_interleave(rep, 1).permute(1, 0, 2).contiguous(), is_causal=True)
    h = X + a.permute(1, 0, 2).reshape(m, hq * dh) @ t(w.wo).T
    hn = F.rms_norm(h, (d,), t(w.mlp_norm), eps)
    y = h + (F.silu(hn @ t(w.w_gate).T) * (hn @ t(w.w_up).T)) @ t(w.w_down).T
    return y.numpy(), hn.numpy()


@pytest.mark.parametrize("hq,hkv", [(4, 2), (2, 2)])
def test_layer_equals_library_composition(hq, hkv):
    rng = np.random.default_rng(hq * 10 + hkv)
    d, dh, f, m = 32, 8, 48, 23
    w = _layer(rng, d, hq, hkv, dh, f)
    x = rng.standard_normal((m, d))
    pos = np.arange(m) + 3
    y, hn = oracle.decoder_layer(x, pos, None, w, [0, m], hq, hkv, dh, 1e-6, 1e4, bf16=False)
    yt, hnt = _torch_layer(x, pos, w, hq, hkv, dh, 1e-6, 1e4)
    np.testing.assert_allclose(y, yt, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(hn, hnt, rtol=1e-11, atol=1e-11)


def test_zero_output_projections_give_identity():
    rng = np.random.default_rng(7)
    d, hq, hkv, dh, f, m = 32, 2, 1, 16, 64, 9
    w = _layer(rng, d, hq, hkv, dh, f)
    w.wo = np.zeros_like(w.wo)
    w.w_down = np.zeros_like(w.w_down)
    x = oracle.round_bf16(rng.standard_normal((m, d)))
    y, _ = oracle.decoder_layer(x, np.arange(m), None, w, [0, m], hq, hkv, dh, 1e-6, 1e6)
    np.testing.assert_array_equal(y, x)


def test_pruned_stack_without_pruning_is_the_full_stack():
    rng = np.random.default_rng(11)
    d, hq, hkv, dh, f, n_layers, gl = 32, 4, 2, 8, 64, 5, 1
    layers = [_layer(rng, d, hq, hkv, dh, f, gated=False) for _ in range(n_layers)]
    for li in range(gl + 1, n_layers):  # gated layers with g = 0, tau = 1
        layers[li].gain = np.zeros(hq)
        layers[li].tau = np.ones(hq)
    gw1, gw2 = rng.standard_normal((16, d)) * 0.2, rng.standard_normal(16) * 0.3
    x0 = oracle.round_bf16(rng.standard_normal((40, d)))
    seg = ([0, 40], [0], [34], [34])  # K = whole document
    y, idx, offs, s = oracle.pruned_stack(x0, layers, gl, gw1, gw2, *seg, hq, hkv, dh)
    assert idx.tolist() == list(range(40))
    x = x0
    for li in range(n_layers):
        x, _ = oracle.decoder_layer(x, np.arange(40), None, layers[li], [0, 40], hq, hkv, dh, 1e-6, 1e6)
    np.testing.assert_array_equal(y, x)
    # with pruning the kept rows are the selector's and their count is K + question
    y2, idx2, offs2, _ = oracle.pruned_stack(x0, layers, gl, gw1, gw2, [0, 40], [0], [34], [10], hq, hkv, dh)
    assert idx2.size == 16 and y2.shape == (16, d) and np.all(idx2[-6:] == np.arange(34, 40))


def _torch_masked_layer(x, pos, w, hq, hkv, dh, eps, theta, seg_id, key_kept, key_score):
    """One layer over every token (float64 torch routines) where a query row r attends key t only if t <= r in
    the same prompt and t is kept (every row also sees itself, which only matters for pruned rows, whose outputs
    are never compared); with key_score the logit gets gain_h * s_t and q.k is scaled by tau_h.  Written
    independently of the oracle's compaction: no row is moved, the rotary angle is the token's own position."""
    F = torch.nn.functional
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    X = t(x)
    m, d = X.shape
    xn = F.rms_norm(X, (d,), t(w.attn_norm), eps)
    q = (xn @ t(w.wq).T).reshape(m, hq, dh)
    k = (xn @ t(w.wk).T).reshape(m, hkv, dh)
    v = (xn @ t(w.wv).T).reshape(m, hkv, dh)
    half = dh // 2
    inv = theta ** (-torch.arange(half, dtype=torch.float64) * 2 / dh)
    ang = t(pos)[:, None] * inv[None, :]
    cos = torch.cat([ang.cos(), ang.cos()], -1)[:, None, :]
    sin = torch.cat([ang.sin(), ang.sin()], -1)[:, None, :]
    rot = lambda z: torch.cat([-z[..., half:], z[..., :half]], -1)
    q = q * cos + rot(q) * sin
    k = k * cos + rot(k) * sin
    r_ = torch.arange(m)
    sid = torch.from_numpy(np.asarray(seg_id))
    vis = (r_[None, :] <= r_[:, None]) & (sid[None, :] == sid[:, None])
    vis &= torch.from_numpy(np.asarray(key_kept))[None, :] | torch.eye(m, dtype=torch.bool)
    bias = torch.zeros(hq, m, m, dtype=torch.float64)
    if key_score is not None:
        bias += t(w.gain)[:, None, None] * t(key_score)[None, None, :]
        q = q * t(w.tau)[None, :, None]
    mask = torch.where(vis[None], bias, torch.tensor(-math.inf, dtype=torch.float64))
    rep = hq // hkv
    a = F.scaled_dot_product_attention(q.permute(1, 0, 2), k.repeat_interleave(rep, 1).permute(1, 0, 2).contiguous(),
                                       v.repeat_interleave(rep, 1).permute(1, 0, 2).contiguous(), attn_mask=mask)
    h = X + a.permute(1, 0, 2).reshape(m, hq * dh) @ t(w.wo).T
    hn = F.rms_norm(h, (d,), t(w.mlp_norm), eps)
    y = h + (F.silu(hn @ t(w.w_gate).T) * (hn @ t(w.w_up).T)) @ t(w.w_down).T
    return y.numpy(), hn.numpy()


@pytest.mark.parametrize("gate_bias", [False, True])
def test_pruned_stack_equals_masked_full_length_forward(gate_bias):
    """[reading] §4.1 (three-stage forward; the temperature's p_i is the original position, m_i the kept rank):
    above the gate, processing only the kept rows at their original positions is the same as processing every
    token with the pruned keys masked out.  Two prompts, a kept set far from the identity (K well below the
    document), positions restarting per prompt.  With the gate bias off (g = 0) the gated layers are plain causal
    attention over the kept keys; with it on, each kept key adds gain_h * s_t.  Using the kept rank instead of the
    position for the rotary angle, or another token's score as the bias, breaks the equality."""
    rng = np.random.default_rng(41)
    d, hq, hkv, dh, f, n_layers, gl = 32, 4, 2, 8, 48, 4, 1
    layers = [_layer(rng, d, hq, hkv, dh, f, gated=li > gl) for li in range(n_layers)]
    if not gate_bias:
        for li in range(gl + 1, n_layers):
            layers[li].gain = np.zeros(hq)
    gw1, gw2 = rng.standard_normal((16, d)) * 0.3, rng.standard_normal(16) * 0.5
    seg_start, doc_begin, doc_end, k_budget = [0, 37, 64], [3, 0], [31, 20], [9, 5]
    n = seg_start[-1]
    x0 = rng.standard_normal((n, d))
    y, idx, offs, s = oracle.pruned_stack(x0, layers, gl, gw1, gw2, seg_start, doc_begin, doc_end, k_budget, hq, hkv,
                                          dh, bf16=False)
    # the kept set is a real pruning: neither all tokens nor a prefix, and kept rank != position somewhere
    assert idx.size == 9 + 9 + 5 + 7
    pos = np.concatenate([np.arange(seg_start[i + 1] - seg_start[i]) for i in range(2)])
    seg_id = np.concatenate([np.full(seg_start[i + 1] - seg_start[i], i) for i in range(2)])
    ranks = np.concatenate([np.arange(offs[i + 1] - offs[i]) for i in range(2)])
    assert np.any(pos[idx] != ranks)
    kept = np.zeros(n, bool)
    kept[idx] = True
    # full-length forward: every token through every layer, pruned keys masked above the gate
    x = x0
    for li in range(n_layers):
        above = li > gl
        x, _ = _torch_masked_layer(x, pos, layers[li], hq, hkv, dh, 1e-6, 1e6, seg_id,
                                   kept if above else np.ones(n, bool), s if above else None)
    np.testing.assert_allclose(y, x[idx], rtol=1e-10, atol=1e-10)
