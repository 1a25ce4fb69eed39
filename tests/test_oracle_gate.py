"""Pins of the oracle's gate (MLP score + sequence RMS normalisation) against
closed forms and invariants, not against itself."""
import math

import numpy as np
import pytest

import oracle
from conftest import floats, golden_lines


def _fixture():
    return dict(ln.split(":", 1) for ln in golden_lines("gate_closed_form.txt"))


def test_closed_form_identity_w1():
    g = _fixture()
    ts = floats(g["raw_t"])
    x = np.array([[t, -t] for t in ts])
    r = oracle.gate_raw_scores(x, np.eye(2), None, np.array([1.0, 1.0]), 0.0)
    np.testing.assert_allclose(r, floats(g["raw_r"]), rtol=0, atol=1e-15)
    b = oracle.sequence_rms_normalize(r, float(g["eps"]))
    np.testing.assert_allclose(b, floats(g["normalized_b"]), rtol=0, atol=1e-15)
    # the tanh approximation is a different function: the erf reading is the one pinned
    assert abs(r[0] - floats(g["tanh_variant_r_t1"])[0]) > 1e-4


def test_antisymmetric_w2_gives_identity():
    g = _fixture()
    ts = floats(g["antisym_t"])
    x = np.array([[t, -t] for t in ts])
    r = oracle.gate_raw_scores(x, np.eye(2), None, np.array([1.0, -1.0]), 0.0)
    np.testing.assert_allclose(r, floats(g["antisym_r"]), rtol=1e-14, atol=1e-14)


def test_nonsquare_selection_w1_and_biases():
    # W1 picks components 0 and 2 of a 3-wide row: a transposed W1 cannot even be applied
    w1 = np.array([[1.0, 0.0, 0.0], [0.0, 0.0, 1.0]])
    x = np.array([[1.0, 99.0, -1.0], [0.0, -7.0, 0.0]])
    r = oracle.gate_raw_scores(x, w1, None, np.array([1.0, 1.0]), 0.0)
    assert r[0] == pytest.approx(math.erf(1 / math.sqrt(2)), abs=1e-15)
    assert r[1] == 0.0
    # b1 = [beta, -beta] on a zero row gives beta erf(beta / sqrt 2); b2 shifts the result
    beta = 2.0
    r = oracle.gate_raw_scores(np.zeros((1, 3)), w1, np.array([beta, -beta]), np.array([1.0, 1.0]), 0.25)
    assert r[0] == pytest.approx(2 * math.erf(math.sqrt(2)) + 0.25, abs=1e-15)
    with pytest.raises(ValueError):
        oracle.gate_raw_scores(x, w1.T, None, np.array([1.0, 1.0]), 0.0)


def test_rms_invariants():
    rng = np.random.default_rng(0)
    r = rng.standard_normal(1000) * 3.0
    eps = 1e-6
    b = oracle.sequence_rms_normalize(r, eps)
    m = np.mean(r * r)
    assert np.mean(b * b) == pytest.approx(m / (m + eps), rel=1e-13)
    # positive rescaling of the MLP output leaves b unchanged (eps = 0), a sign flip flips it
    np.testing.assert_allclose(oracle.sequence_rms_normalize(7.5 * r, 0.0), oracle.sequence_rms_normalize(r, 0.0),
                               rtol=1e-14)
    np.testing.assert_allclose(oracle.sequence_rms_normalize(-r, 0.0), -oracle.sequence_rms_normalize(r, 0.0),
                               rtol=1e-14)
    # eps < 0 disables the normalisation; order is preserved
    np.testing.assert_array_equal(oracle.sequence_rms_normalize(r, -1.0), r)
    assert np.array_equal(np.argsort(b, kind="stable"), np.argsort(r, kind="stable"))
    assert oracle.sequence_rms_normalize(np.zeros(0), eps).size == 0


def test_segments_are_independent_and_non_doc_is_zero():
    rng = np.random.default_rng(1)
    d, h = 8, 5
    w1 = rng.standard_normal((h, d))
    w2 = rng.standard_normal(h)
    a = rng.standard_normal((6, d))
    bb = rng.standard_normal((9, d))
    # segment 0: 2 instruction tokens, doc a, 1 question token; segment 1: doc bb then 3 question tokens
    x = np.concatenate([rng.standard_normal((2, d)), a, rng.standard_normal((1, d)), bb, rng.standard_normal((3, d))])
    seg_start = [0, 9, 21]
    s = oracle.gate_scores(x, w1, None, w2, 0.0, seg_start, [2, 0], [8, 9])
    assert np.all(s[[0, 1, 8, 18, 19, 20]] == 0.0)
    alone_a = oracle.gate_scores(a, w1, None, w2, 0.0, [0, 6], [0], [6])
    alone_b = oracle.gate_scores(bb, w1, None, w2, 0.0, [0, 9], [0], [9])
    np.testing.assert_allclose(s[2:8], alone_a, rtol=1e-14)
    np.testing.assert_allclose(s[9:18], alone_b, rtol=1e-14)
    # the same document in two prompts gets the same normalised scores
    x2 = np.concatenate([a, a])
    s2 = oracle.gate_scores(x2, w1, None, w2, 0.0, [0, 6, 12], [0, 0], [6, 6])
    np.testing.assert_array_equal(s2[:6], s2[6:])
