"""Pins of the oracle's selector: hand-worked cases, the rank definition, a
full stable sort, and the invariants of S = top-K ∪ N."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from conftest import golden_lines
from learned_token_pruning_amd import workloads


def _parse(tok):
    return float(tok)


@pytest.mark.parametrize("line", golden_lines("select_worked.txt"))
def test_worked_cases(line):
    name, docs, extra, k, kept = [p.strip() for p in line.split("|")]
    doc = np.array([_parse(t) for t in docs.split()], dtype=np.float32)
    n_extra = int(extra)
    scores = np.concatenate([doc, np.zeros(n_extra, np.float32)])
    idx, offs = oracle.kept_indices(scores, [0, scores.size], [0], [doc.size], [int(k)])
    expect = [int(t) for t in kept.split()]
    assert idx.tolist() == expect, name
    assert offs.tolist() == [0, len(expect)]
    # the other two formulations agree on every worked case
    kd = int(k)
    assert oracle.select_doc_topk_by_rank(doc, kd).tolist() == oracle.select_doc_topk(doc, kd).tolist()
    assert oracle.select_doc_topk_by_sort(doc, kd).tolist() == oracle.select_doc_topk(doc, kd).tolist()


_vals = st.sampled_from([0.0, -0.0, 1.0, -1.0, 2.5, float("inf"), float("-inf"), float("nan"), 1e-38, -3.0])


@settings(max_examples=300, deadline=None)
@given(st.lists(_vals, min_size=0, max_size=48), st.integers(min_value=0, max_value=60))
def test_threshold_counting_equals_rank_and_sort(vals, k):
    v = np.array(vals, dtype=np.float32)
    a = oracle.select_doc_topk(v, k)
    assert a.tolist() == oracle.select_doc_topk_by_rank(v, k).tolist()
    assert a.tolist() == oracle.select_doc_topk_by_sort(v, k).tolist()


@settings(max_examples=100, deadline=None)
@given(st.lists(st.floats(width=32, allow_nan=False), min_size=1, max_size=64), st.integers(0, 70))
def test_random_floats(vals, k):
    v = np.array(vals, dtype=np.float32)
    assert oracle.select_doc_topk(v, k).tolist() == oracle.select_doc_topk_by_sort(v, k).tolist()


def _check_invariants(scores, seg, idx, offs):
    for i in range(seg.n_seg):
        a, b = seg.seg_start[i], seg.seg_start[i + 1]
        lo, hi = a + seg.doc_begin[i], a + seg.doc_end[i]
        kept = idx[offs[i]:offs[i + 1]]
        n_doc = hi - lo
        keff = min(seg.k_budget[i], n_doc)
        assert kept.size == keff + (b - a - n_doc) == oracle.kept_count(n_doc, b - a - n_doc, seg.k_budget[i])
        assert np.all(np.diff(kept) > 0)
        assert np.all((kept >= a) & (kept < b))
        other = np.concatenate([np.arange(a, lo), np.arange(hi, b)])
        assert np.isin(other, kept).all()
        dk = kept[(kept >= lo) & (kept < hi)]
        dropped = np.setdiff1d(np.arange(lo, hi), dk)
        if dk.size and dropped.size:
            kmin = scores[dk].astype(np.float64).min()
            dmax = scores[dropped].astype(np.float64).max()
            assert kmin >= dmax
            if kmin == dmax:
                assert dk[scores[dk] == kmin].max() < dropped[scores[dropped] == dmax].min()


def test_invariants_on_mixture_scores():
    seg = workloads.single_segment(4000, 64, 0)
    s = workloads.mixture_scores(3, seg, k_marks=(100, 1000))
    for k in (0, 1, 100, 1000, 3999, 4000, 5000):
        sk = seg.with_budget(k)
        idx, offs = oracle.kept_indices(s, sk.seg_start, sk.doc_begin, sk.doc_end, sk.k_budget)
        _check_invariants(s, sk, idx, offs)


def test_planted_ties_straddle_the_boundary():
    seg = workloads.single_segment(5000, 64, 0)
    s = workloads.mixture_scores(3, seg, k_marks=(1000,))
    doc = s[:5000].astype(np.float64)
    t = np.sort(doc)[::-1][999]
    assert (doc > t).sum() < 1000 < (doc >= t).sum()
    kept = oracle.select_doc_topk(doc, 1000)
    ties = np.flatnonzero(doc == t)
    need = 1000 - int((doc > t).sum())
    assert np.isin(ties[:need], kept).all() and not np.isin(ties[need:], kept).any()


def test_all_equal_scores_keep_first_k():
    # a zero-initialised gate outputs 0 for every token: the selector keeps the first K documents
    doc = np.zeros(50, np.float32)
    assert oracle.select_doc_topk(doc, 7).tolist() == list(range(7))


def test_segments_are_independent():
    rng = np.random.default_rng(5)
    seg = workloads.random_segments(rng, 12, 80)
    s = workloads.mixture_scores(7, seg)
    idx, offs = oracle.kept_indices(s, seg.seg_start, seg.doc_begin, seg.doc_end, seg.k_budget)
    _check_invariants(s, seg, idx, offs)
    for i in range(seg.n_seg):
        a, b = seg.seg_start[i], seg.seg_start[i + 1]
        one, _ = oracle.kept_indices(s[a:b], [0, b - a], [seg.doc_begin[i]], [seg.doc_end[i]], [seg.k_budget[i]])
        assert (one + a).tolist() == idx[offs[i]:offs[i + 1]].tolist()


def test_negative_budget_rejected():
    with pytest.raises(ValueError):
        oracle.kept_indices(np.zeros(4, np.float32), [0, 4], [0], [4], [-1])
    with pytest.raises(ValueError):
        oracle.kept_count(3, 1, -2)
