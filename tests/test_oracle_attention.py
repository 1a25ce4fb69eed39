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
