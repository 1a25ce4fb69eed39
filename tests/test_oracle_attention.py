"""Pins of the oracle's token-gated attention: a hand-worked example, the
reduction to a library scaled-dot-product attention (with the gate as an
additive float mask and the temperature folded into q), and limits."""
import math

import numpy as np
import pytest
import torch

import oracle
from conftest import floats, golden_lines

LN2 = math.log(2.0)


def _worked_inputs(ln2):
    q = np.ones((4, 1, 1))
    k = np.array([0.0, ln2, 0.0, 0.0]).reshape(4, 1, 1)
    v = np.array([8.0, 0.0, 4.0, 0.0]).reshape(4, 1, 1)
    s = np.array([0.0, 0.0, ln2, 0.0])
    return q, k, v, s


@pytest.mark.parametrize("line", golden_lines("attention_worked.txt"))
def test_worked_example(line):
    lhs, rhs = line.split("|")
    parts = lhs.split()
    tol = 1e-12
    ln2 = LN2
    if parts[0] == "bf16":
        parts = parts[1:]
        ln2 = 0.69140625
        tol = 1e-6
    tau, g = float(parts[0]), float(parts[1])
    q, k, v, s = _worked_inputs(ln2)
    o = oracle.gated_attention(q, k, v, s, np.array([tau]), np.array([g]), [0, 4])
    np.testing.assert_allclose(o[:, 0, 0], floats(rhs), rtol=0, atol=tol)


def _sdpa_ref(q, k, v, tau, bias_mask):
    """torch's scaled_dot_product_attention (float64, CPU) with K/V heads repeated."""
    m, hq, d = q.shape
    group = hq // k.shape[1]
    qt = torch.from_numpy(q * tau[None, :, None]).permute(1, 0, 2)
    kt = torch.from_numpy(np.repeat(k, group, axis=1)).permute(1, 0, 2).contiguous()
    vt = torch.from_numpy(np.repeat(v, group, axis=1)).permute(1, 0, 2).contiguous()
    if bias_mask is None:
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    else:
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(bias_mask))
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("hq,hkv", [(4, 2), (3, 3), (6, 1)])
def test_reduces_to_causal_softmax_attention(hq, hkv):
    rng = np.random.default_rng(hq * 10 + hkv)
    m, d = 37, 16
    q, k, v = (rng.standard_normal((m, h, d)) for h in (hq, hkv, hkv))
    s = rng.standard_normal(m)
    ones = np.ones(hq)
    o = oracle.gated_attention(q, k, v, s, ones, np.zeros(hq), [0, m])
    np.testing.assert_allclose(o, _sdpa_ref(q, k, v, ones, None), rtol=1e-12, atol=1e-12)
    o2 = oracle.gated_attention(q, k, v, None, None, None, [0, m])
    np.testing.assert_allclose(o2, o, rtol=1e-13, atol=1e-13)


def test_gate_and_temperature_equal_library_attention_with_float_mask():
    rng = np.random.default_rng(3)
    m, hq, hkv, d = 29, 4, 2, 8
    q, k, v = (rng.standard_normal((m, h, d)) for h in (hq, hkv, hkv))
    s = rng.standard_normal(m)
    tau = rng.uniform(0.8, 1.2, hq)
    gain = rng.uniform(0.5, 1.5, hq)
    o = oracle.gated_attention(q, k, v, s, tau, gain, [0, m])
    causal = np.tril(np.ones((m, m), bool))
    for h in range(hq):
        mask = np.where(causal, gain[h] * s[None, :], -np.inf)
        ref = _sdpa_ref(q[:, h:h + 1], k[:, h // 2:h // 2 + 1], v[:, h // 2:h // 2 + 1], tau[h:h + 1], mask)
        np.testing.assert_allclose(o[:, h], ref[:, 0], rtol=1e-12, atol=1e-12)


def test_segments_are_block_diagonal_and_rows_subset():
    rng = np.random.default_rng(4)
    offs = [0, 5, 5, 17, 18]
    m, hq, hkv, d = 18, 2, 1, 4
    q, k, v = (rng.standard_normal((m, h, d)) for h in (hq, hkv, hkv))
    s = rng.standard_normal(m)
    tau, gain = np.array([1.1, 0.9]), np.array([0.7, 1.3])
    o = oracle.gated_attention(q, k, v, s, tau, gain, offs)
    for a, b in zip(offs[:-1], offs[1:]):
        if b > a:
            np.testing.assert_allclose(
                o[a:b], oracle.gated_attention(q[a:b], k[a:b], v[a:b], s[a:b], tau, gain, [0, b - a]), rtol=1e-14)
    rows = np.array([17, 3, 10])
    np.testing.assert_allclose(oracle.gated_attention(q, k, v, s, tau, gain, offs, rows=rows), o[rows], rtol=1e-14)
    # a one-row prompt returns its own value row
    np.testing.assert_allclose(o[17], np.repeat(v[17], hq, axis=0), rtol=1e-15)


def test_large_gain_selects_highest_score_key():
    rng = np.random.default_rng(6)
    m, d = 12, 4
    q, k, v = (rng.standard_normal((m, 1, d)) for _ in range(3))
    s = rng.permutation(m).astype(np.float64)
    o = oracle.gated_attention(q, k, v, s, np.array([1.0]), np.array([200.0]), [0, m])
    for r in range(m):
        best = int(np.argmax(s[:r + 1]))
        np.testing.assert_allclose(o[r, 0], v[best, 0], atol=1e-9)


# ----------------------------------------------------------------------------- per-query temperature


def test_softplus_closed_forms():
    assert oracle.softplus(np.array([0.0]))[0] == pytest.approx(LN2, abs=1e-15)
    x = np.array([-30.0, -2.5, -0.1, 0.3, 4.0, 40.0, 800.0])
    # softplus(x) - softplus(-x) = x, softplus(x) > max(x, 0), and e^softplus(x) - 1 = e^x
    np.testing.assert_allclose(oracle.softplus(x) - oracle.softplus(-x), x, rtol=1e-14, atol=1e-14)
    assert np.all(oracle.softplus(x[:5]) > np.maximum(x[:5], 0.0)) and oracle.softplus(x[-1:])[0] == 800.0
    small = x[x < 5]
    np.testing.assert_allclose(np.expm1(oracle.softplus(small)), np.exp(small), rtol=1e-13)


def test_query_temperature_ranks_restart_per_prompt():
    sig = np.array([0.0, 2.0])
    pos = np.array([0, 4, 9, 2, 3])  # prompt 0 keeps positions 0, 4, 9; prompt 1 keeps 2, 3
    t = oracle.query_temperature(sig, pos, [0, 3, 3, 5])
    sp = np.log1p(np.exp(sig))
    ranks = np.array([1, 2, 3, 1, 2])
    orig = np.array([1, 5, 10, 3, 4])
    for r in range(5):
        want = 0.0 if ranks[r] == 1 else math.log(ranks[r]) / math.log(orig[r])
        np.testing.assert_allclose(t[r], sp * want, rtol=1e-14, atol=0)
    # kept rows in original order: rank <= position, so 0 <= tau <= softplus(sigma)
    assert np.all(t >= 0) and np.all(t <= sp[None, :] + 1e-15)


def test_query_temperature_is_identity_without_pruning():
    """Nothing pruned: every query keeps all its keys (m_i = p_i), the
    recalibration factor is 1, and the attention equals the per-head form
    with tau_h = softplus(sigma_h)."""
    rng = np.random.default_rng(11)
    offs = [0, 9, 10, 31]
    m, hq, hkv, d = 31, 4, 2, 8
    q, k, v = (rng.standard_normal((m, h, d)) for h in (hq, hkv, hkv))
    s = rng.standard_normal(m)
    sigma = rng.uniform(-1.0, 1.5, hq)
    gain = rng.uniform(0.5, 1.5, hq)
    pos = np.concatenate([np.arange(b - a) for a, b in zip(offs[:-1], offs[1:])])
    t = oracle.query_temperature(sigma, pos, offs)
    first = np.isin(np.arange(m), offs[:-1])
    np.testing.assert_allclose(t[~first], np.broadcast_to(oracle.softplus(sigma), (m - 3, hq)), rtol=1e-14)
    o = oracle.gated_attention(q, k, v, s, t, gain, offs)
    np.testing.assert_allclose(o, oracle.gated_attention(q, k, v, s, oracle.softplus(sigma), gain, offs),
                               rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("g", [0.0, 1.0])
def test_query_temperature_worked_example(g):
    """Three kept tokens at original positions 0, 3, 7 (1 head, D = 1), with
    softplus(sigma) = 2, q = 1, k = [0, ln2, 0], v = [6, 0, 3], s = [0, 0, ln2].
    Worked by hand: tau = [0, 2 ln2/ln4, 2 ln3/ln8] = [0, 1, (2/3) log2 3], so
    row 1 weighs exp([0, ln2]) = [1, 2]; row 2 weighs [1, 2^tau_2, 2^g] with
    2^tau_2 = 3^(2/3) (the bias is not scaled by the temperature)."""
    sigma = np.array([math.log(math.expm1(2.0))])
    pos = np.array([0, 3, 7])
    t = oracle.query_temperature(sigma, pos, [0, 3])
    np.testing.assert_allclose(t[:, 0], [0.0, 1.0, 2.0 * math.log(3.0) / math.log(8.0)], rtol=1e-14)
    q = np.ones((3, 1, 1))
    k = np.array([0.0, LN2, 0.0]).reshape(3, 1, 1)
    v = np.array([6.0, 0.0, 3.0]).reshape(3, 1, 1)
    s = np.array([0.0, 0.0, LN2])
    o = oracle.gated_attention(q, k, v, s, t, np.array([g]), [0, 3])[:, 0, 0]
    c = 3.0 ** (2.0 / 3.0)
    w2 = 2.0 ** g
    np.testing.assert_allclose(o, [6.0, 2.0, (6.0 + 3.0 * w2) / (1.0 + c + w2)], rtol=1e-13)


def test_query_temperature_vanishing_leaves_the_bias_softmax():
    """softplus(sigma) -> 0: the logits reduce to the gate bias, so each row is
    the causal softmax(g s)-weighted mean of v, whatever q and k are."""
    rng = np.random.default_rng(12)
    m, d = 14, 4
    q, k, v = (rng.standard_normal((m, 1, d)) * 5 for _ in range(3))
    s = rng.standard_normal(m)
    pos = np.sort(rng.choice(100, m, replace=False))
    t = oracle.query_temperature(np.array([-80.0]), pos, [0, m])
    o = oracle.gated_attention(q, k, v, s, t, np.array([1.3]), [0, m])
    for r in range(m):
        w = [math.exp(1.3 * s[j]) for j in range(r + 1)]
        want = sum(w[j] * v[j, 0] for j in range(r + 1)) / sum(w)
        np.testing.assert_allclose(o[r, 0], want, rtol=1e-12)


# ----------------------------------------------------------------------------- decode


def test_decode_equals_prefill_row_by_row():
    """Causal prefill is decode applied to every prefix: row r of the prefill
    oracle equals a decode step of q_r over the cache rows 0 .. r."""
    rng = np.random.default_rng(21)
    m, hq, hkv, d = 23, 4, 2, 8
    q, k, v = (rng.standard_normal((m, h, d)) for h in (hq, hkv, hkv))
    s = rng.standard_normal(m)
    tau = rng.uniform(0.8, 1.2, hq)
    gain = rng.uniform(0.5, 1.5, hq)
    pre = oracle.gated_attention(q, k, v, s, tau, gain, [0, m])
    cap = m + 5
    kc = np.zeros((m, cap, hkv, d))
    vc = np.zeros((m, cap, hkv, d))
    sc = np.zeros((m, cap))
    kc[:, :m], vc[:, :m], sc[:, :m] = k[None], v[None], s[None]
    kc[:, m:] = 1e3  # rows past a sequence's length never count
    dec = oracle.gated_attention_decode(q, kc, vc, sc, tau, gain, np.arange(1, m + 1))
    np.testing.assert_allclose(dec, pre, rtol=1e-13, atol=1e-13)
    # a per-query temperature row gives the same as the per-head form when it repeats tau
    dec2 = oracle.gated_attention_decode(q, kc, vc, sc, np.tile(tau, (m, 1)), gain, np.arange(1, m + 1))
    np.testing.assert_allclose(dec2, dec, rtol=1e-15)


@pytest.mark.parametrize("g,want", [(0.0, (8.0 + 3 * 4.0) / 4), (1.0, (2 * 8.0 + 3 * 4.0) / 5)])
def test_decode_two_key_closed_form(g, want):
    """q = 1, D = 1, k = [0, ln 3], v = [8, 4], s = [ln 2, 0], tau = 1: by hand
    the weights are [1, 3] / 4 without the gate and [2, 3] / 5 with g = 1."""
    q = np.ones((1, 1, 1))
    kc = np.array([0.0, math.log(3.0)]).reshape(1, 2, 1, 1)
    vc = np.array([8.0, 4.0]).reshape(1, 2, 1, 1)
    s = np.array([[LN2, 0.0]])
    o = oracle.gated_attention_decode(q, kc, vc, s, np.array([1.0]), np.array([g]), [2])
    assert o[0, 0, 0] == pytest.approx(want, rel=1e-14)


def test_decode_empty_and_single_key():
    rng = np.random.default_rng(22)
    q = rng.standard_normal((3, 4, 8))
    kc, vc = rng.standard_normal((2, 3, 5, 2, 8))
    s = rng.standard_normal((3, 5))
    o = oracle.gated_attention_decode(q, kc, vc, s, None, np.ones(4), [0, 1, 5])
    assert np.all(o[0] == 0.0)
    np.testing.assert_allclose(o[1], np.repeat(vc[1, 0], 2, axis=0), rtol=1e-15)
    assert np.all(np.isfinite(o[2]))


# ----------------------------------------------------------------------------- backward


def _loss(q, k, v, s, tau, gain, offs, w):
    return float((oracle.gated_attention(q, k, v, s, tau, gain, offs) * w).sum())


def test_backward_matches_finite_differences():
    """Every gradient against central differences of the forward (step 1e-6,
    float64) on a two-prompt GQA case: the loss is sum(O * W) for a fixed W,
    so dout = W."""
    rng = np.random.default_rng(31)
    offs = [0, 5, 9]
    m, hq, hkv, d = 9, 4, 2, 3
    q, k, v = (rng.standard_normal((m, h, d)) for h in (hq, hkv, hkv))
    s = rng.standard_normal(m)
    tau = rng.uniform(0.6, 1.4, hq)
    gain = rng.uniform(0.5, 1.5, hq)
    w = rng.standard_normal((m, hq, d))
    g = oracle.gated_attention_backward(q, k, v, s, tau, gain, offs, w)
    eps = 1e-6
    args = {"q": q, "k": k, "v": v, "s": s, "gain": gain, "tau": tau}
    names = {"q": "dq", "k": "dk", "v": "dv", "s": "ds", "gain": "dgain", "tau": "dtau"}
    for name, arr in args.items():
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            plus, minus = dict(args), dict(args)
            plus[name] = arr.copy()
            minus[name] = arr.copy()
            plus[name][idx] += eps
            minus[name][idx] -= eps
            num[idx] = (_loss(plus["q"], plus["k"], plus["v"], plus["s"], plus["tau"], plus["gain"], offs, w)
                        - _loss(minus["q"], minus["k"], minus["v"], minus["s"], minus["tau"], minus["gain"], offs,
                                w)) / (2 * eps)
        np.testing.assert_allclose(g[names[name]], num, rtol=1e-6, atol=1e-7, err_msg=name)


def test_backward_matches_torch_autograd():
    """Against torch autograd (float64, CPU) through a forward written with
    torch ops: logits tau q k^T / sqrt(D) + g s plus a causal -inf mask."""
    rng = np.random.default_rng(32)
    m, hq, hkv, d = 21, 4, 2, 8
    group = hq // hkv
    q, k, v = (rng.standard_normal((m, h, d)) for h in (hq, hkv, hkv))
    s = rng.standard_normal(m)
    tau = rng.uniform(0.6, 1.4, hq)
    gain = rng.uniform(0.5, 1.5, hq)
    dout = rng.standard_normal((m, hq, d))
    tq, tk, tv, ts, tt, tg = (torch.tensor(a, requires_grad=True) for a in (q, k, v, s, tau, gain))
    kk = tk.repeat_interleave(group, dim=1).permute(1, 0, 2)
    vv = tv.repeat_interleave(group, dim=1).permute(1, 0, 2)
    z = tt[:, None, None] * (tq.permute(1, 0, 2) @ kk.transpose(1, 2)) / math.sqrt(d) + tg[:, None, None] * ts[None,
                                                                                                               None, :]
    mask = torch.triu(torch.ones(m, m, dtype=torch.bool), diagonal=1)
    z = z.masked_fill(mask, float("-inf"))
    o = (torch.softmax(z, dim=-1) @ vv).permute(1, 0, 2)
    (o * torch.from_numpy(dout)).sum().backward()
    g = oracle.gated_attention_backward(q, k, v, s, tau, gain, [0, m], dout)
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv), ("ds", ts), ("dtau", tt), ("dgain", tg)):
        np.testing.assert_allclose(g[name], t.grad.numpy(), rtol=1e-10, atol=1e-11, err_msg=name)


def test_logsumexp_closed_form_and_normalisation():
    rng = np.random.default_rng(33)
    offs = [0, 6, 17]
    m, hq, hkv, d = 17, 2, 1, 4
    q, k = rng.standard_normal((m, hq, d)), rng.standard_normal((m, hkv, d))
    # uniform logits (tau = 0, no bias): ln(number of visible keys)
    lse0 = oracle.attention_logsumexp(q, k, None, np.zeros(hq), None, offs)
    r = np.concatenate([np.arange(6), np.arange(11)]) + 1
    np.testing.assert_allclose(lse0, np.log(r)[:, None].repeat(hq, 1), rtol=1e-14)
    # with temperature and bias: exp(z - lse) sums to 1 over the visible keys
    s = rng.standard_normal(m)
    tau, gain = np.array([1.3, 0.7]), np.array([0.9, 1.4])
    lse = oracle.attention_logsumexp(q, k, s, tau, gain, offs)
    for a, b in zip(offs[:-1], offs[1:]):
        for row in range(a, b):
            for h in range(hq):
                z = [tau[h] * float(q[row, h] @ k[t, 0]) / 2.0 + gain[h] * s[t] for t in range(a, row + 1)]
                assert sum(math.exp(x - lse[row, h]) for x in z) == pytest.approx(1.0, rel=1e-13)
