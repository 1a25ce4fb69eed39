"""Reference (float64, CPU) of the TokenGate gate, selector, compaction and
token-gated attention.  TEST INFRASTRUCTURE: see the package docstring.

Every function follows a passage of the pages; where the pages leave a step
open the plain reading used here is stated in the docstring.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np
from scipy.special import erf

# ----------------------------------------------------------------------------
# Gate module  ([reading] §4.1 component one; [news] "可学习 token 剪枝如何工作")
# ----------------------------------------------------------------------------


def gelu_erf(u: np.ndarray) -> np.ndarray:
    """Exact (erf) GELU: u * Phi(u) = 0.5 u (1 + erf(u / sqrt 2)).

    The pages name only "a small MLP"; the activation is not stated.  Reading:
    the exact erf form.  Pinned by the closed form GELU(x) + GELU(-x) =
    x erf(x / sqrt 2) (tests/golden/gate_closed_form.txt).
    """
    u = np.asarray(u, dtype=np.float64)
    return 0.5 * u * (1.0 + erf(u / math.sqrt(2.0)))


def gate_raw_scores(x_doc: np.ndarray, w1: np.ndarray, b1: Optional[np.ndarray], w2: np.ndarray,
                    b2: float) -> np.ndarray:
    """Scalar score of every prunable token from its hidden row:
    r_j = w2 . GELU(W1 x_j + b1) + b2  ([reading] §4.1 component one: a small
    MLP reads each prunable token's normalised post-attention residual and
    outputs one scalar).

    x_doc [n, d], w1 [h, d], b1 [h] or None, w2 [h]; all float64.
    Pinned by tests/golden/gate_closed_form.txt (identity W1) and by a
    brute-force per-row loop in the tests.
    """
    x_doc = np.asarray(x_doc, dtype=np.float64)
    u = x_doc @ np.asarray(w1, dtype=np.float64).T
    if b1 is not None:
        u = u + np.asarray(b1, dtype=np.float64)[None, :]
    return gelu_erf(u) @ np.asarray(w2, dtype=np.float64) + float(b2)


def sequence_rms_normalize(r: np.ndarray, eps: float) -> np.ndarray:
    """b_j = r_j / sqrt(mean_{j in P} r_j^2 + eps): the MLP output is
    RMS-normalised along the sequence ([reading] §4.1 component one).

    Reading: over the prunable tokens of one prompt only, no learnable weight
    (a scalar weight would be absorbed by the per-head gain).  eps < 0 means
    "no normalisation" (b = r).  An empty document returns an empty array.
    Pinned by the invariant mean(b^2) = 1 - eps/(mean r^2 + eps) and the
    closed-form fixture.
    """
    r = np.asarray(r, dtype=np.float64)
    if eps < 0 or r.size == 0:
        return r.copy()
    rho = math.sqrt(float(np.mean(r * r)) + eps)
    return r / rho


def gate_scores(x: np.ndarray, w1: np.ndarray, b1: Optional[np.ndarray], w2: np.ndarray, b2: float,
                seg_start: Sequence[int], doc_begin: Sequence[int], doc_end: Sequence[int],
                eps: float = 1e-6) -> np.ndarray:
    """Score s of every token of a packed batch.

    Prunable (document) tokens get the RMS-normalised MLP score b_j; every
    other token (instruction, question) gets exactly 0 and is exempt
    ([reading] §4.1 component one: non-prunable tokens have a fixed score of 0).
    """
    n = int(seg_start[-1])
    s = np.zeros(n, dtype=np.float64)
    for i in range(len(doc_begin)):
        lo = int(seg_start[i]) + int(doc_begin[i])
        hi = int(seg_start[i]) + int(doc_end[i])
        if hi <= lo:
            continue
        r = gate_raw_scores(x[lo:hi], w1, b1, w2, b2)
        s[lo:hi] = sequence_rms_normalize(r, eps)
    return s


# ----------------------------------------------------------------------------
# Top-K selector  ([reading] §3.1 and §4.1: S = top-K(b_j) ∪ N, |S ∩ P| = K)
# ----------------------------------------------------------------------------


def kept_count(n_doc: int, n_other: int, k: int) -> int:
    """|S| = min(K, |P|) + |N|.  Reading of the budget
    ("max_kept_prefill_tokens" in [news] "如何部署 TokenGate？"): a budget above
    the document length keeps the whole document; a negative budget is an error."""
    if k < 0:
        raise ValueError("negative budget")
    return min(k, n_doc) + n_other


def _better(si: float, i: int, sj: float, j: int) -> bool:
    """Strict total order used by the selector: higher score first, lower index
    among equal scores.  IEEE comparison, so -0.0 == +0.0.  NaN ranks below
    every number (including -inf); NaNs among themselves by index."""
    ni, nj = math.isnan(si), math.isnan(sj)
    if ni and nj:
        return i < j
    if ni:
        return False
    if nj:
        return True
    if si != sj:
        return si > sj
    return i < j


def select_doc_topk_by_rank(doc_scores: np.ndarray, k: int) -> np.ndarray:
    """Definition by rank, O(n^2): keep j iff
    #{i : i better than j} < min(K, n).  Returns ascending local indices."""
    v = [float(x) for x in np.asarray(doc_scores, dtype=np.float64)]
    n = len(v)
    keff = min(k, n)
    kept = []
    for j in range(n):
        rank = sum(1 for i in range(n) if i != j and _better(v[i], i, v[j], j))
        if rank < keff:
            kept.append(j)
    return np.asarray(kept, dtype=np.int64)


def select_doc_topk_by_sort(doc_scores: np.ndarray, k: int) -> np.ndarray:
    """Brute force: full stable sort by (score descending, index ascending)
    with NaN last, first min(K, n), returned ascending."""
    v = np.asarray(doc_scores, dtype=np.float64)
    n = v.size
    keff = min(k, n)
    key = [(1 if math.isnan(x) else 0, 0.0 if math.isnan(x) else -x, j) for j, x in enumerate(v.tolist())]
    order = sorted(range(n), key=lambda j: key[j])
    return np.sort(np.asarray(order[:keff], dtype=np.int64))


def select_doc_topk(doc_scores: np.ndarray, k: int) -> np.ndarray:
    """Threshold counting (linear after one sort of the values): let T be the
    K_eff-th largest value; keep every score > T and, among the scores equal
    to T, the K_eff - #{> T} lowest indices.  Equivalent to the rank
    definition; pinned against it and against a full stable sort in the tests."""
    v = np.asarray(doc_scores, dtype=np.float64)
    n = v.size
    keff = min(k, n)
    if keff <= 0:
        return np.zeros(0, dtype=np.int64)
    isnan = np.isnan(v)
    valid = v[~isnan]
    if keff > valid.size:
        keep = ~isnan
        need = keff - valid.size
        nan_idx = np.flatnonzero(isnan)[:need]
        keep[nan_idx] = True
        return np.flatnonzero(keep).astype(np.int64)
    t = np.sort(valid)[::-1][keff - 1]
    gt = (~isnan) & (v > t)
    eq = (~isnan) & (v == t)
    need = keff - int(gt.sum())
    take_eq = eq & (np.cumsum(eq) <= need)
    return np.flatnonzero(gt | take_eq).astype(np.int64)


def kept_indices(scores: np.ndarray, seg_start: Sequence[int], doc_begin: Sequence[int],
                 doc_end: Sequence[int], k_budget: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """Kept set of every prompt of a packed batch, as ascending global token
    indices: S = top-K(doc scores) ∪ (all non-document tokens)
    ([reading] §4.1: S = top-K(b_j) ∪ N; [news]: the question is never pruned).

    Returns (kept_idx [M] int64, kept_offsets [n_seg + 1] int64).
    """
    scores = np.asarray(scores)
    out = []
    offs = [0]
    for i in range(len(doc_begin)):
        a = int(seg_start[i])
        b = int(seg_start[i + 1])
        lo, hi = a + int(doc_begin[i]), a + int(doc_end[i])
        if int(k_budget[i]) < 0:
            raise ValueError("negative budget")
        doc_keep = select_doc_topk(scores[lo:hi], int(k_budget[i])) + lo
        keep = np.concatenate([np.arange(a, lo), doc_keep, np.arange(hi, b)]).astype(np.int64)
        out.append(keep)
        offs.append(offs[-1] + keep.size)
    idx = np.concatenate(out) if out else np.zeros(0, np.int64)
    return idx, np.asarray(offs, dtype=np.int64)


# ----------------------------------------------------------------------------
# Compaction  ([reading] §4.1: pruned tokens never enter the upper layers and
# never get KV entries there; [news] "剪枝前向")
# ----------------------------------------------------------------------------


def compact_rows(rows: np.ndarray, kept_idx: np.ndarray) -> np.ndarray:
    """out[r] = rows[kept_idx[r]]: the kept rows, in original order, bit for bit."""
    return np.asarray(rows)[np.asarray(kept_idx, dtype=np.int64)]


# ----------------------------------------------------------------------------
# Token-gated attention  ([reading] §4.1 component two; [insight] and [news]:
# the kept token's score becomes a logit bias, refined by a per-head gain and
# a temperature)
# ----------------------------------------------------------------------------


def gated_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, s: Optional[np.ndarray],
                    tau: Optional[np.ndarray], gain: Optional[np.ndarray], kept_offsets: Sequence[int],
                    rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Causal token-gated GQA attention over the kept rows.

    For query head h (key/value head c = h // (Hq / Hkv)) and kept row r of a
    prompt, over the kept rows t <= r of the same prompt:
        z_rt = tau_h * (q_r . k_t) / sqrt(D) + g_h * s_t
        O[r, h] = sum_t softmax_t(z_r.) v_t
    The pages write the weights as exp(z)·g_j / sum exp(z)·g_j' with
    g_j = softmax(b_j) ([reading] §4.1 component two), i.e. the score enters
    as an additive logit bias; the per-(layer, head) gain multiplies it and the
    temperature rescales q.k (refinements one and two).  The per-head
    constant tau_h is the reading used here; a [M, Hq] array instead gives
    every kept row its own temperature (see query_temperature).  tau None
    -> 1, gain None or s None -> no bias.

    q [M, Hq, D], k/v [M, Hkv, D], s [M]; float64.  ``rows`` optionally
    restricts the computation to those global kept-row indices (returned in
    that order).  Accumulation in float64.
    Pinned by the hand-worked 4-token fixture and by the reduction to plain
    causal softmax attention (tau = 1, g = 0).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    m_total, hq, dh = q.shape
    hkv = k.shape[1]
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    group = hq // hkv
    tau = np.ones(hq) if tau is None else np.asarray(tau, dtype=np.float64)
    if tau.ndim == 1:
        tau = np.broadcast_to(tau[None, :], (m_total, hq))
    use_bias = s is not None and gain is not None
    if use_bias:
        s = np.asarray(s, dtype=np.float64)
        gain = np.asarray(gain, dtype=np.float64)
    scale = 1.0 / math.sqrt(dh)
    offs = [int(o) for o in kept_offsets]
    if rows is None:
        rows = np.arange(m_total)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, hq, dh), dtype=np.float64)
    seg_of = np.searchsorted(np.asarray(offs[1:]), rows, side="right")
    for si in np.unique(seg_of):
        a, b = offs[si], offs[si + 1]
        sel = np.flatnonzero(seg_of == si)
        r_loc = rows[sel] - a
        nk = int(r_loc.max()) + 1
        causal = np.arange(nk)[None, :] <= r_loc[:, None]
        for h in range(hq):
            c = h // group
            z = tau[a + r_loc, h][:, None] * (q[a + r_loc, h, :] @ k[a:a + nk, c, :].T) * scale
            if use_bias:
                z = z + gain[h] * s[a:a + nk][None, :]
            z = np.where(causal, z, -np.inf)
            z = z - z.max(axis=1, keepdims=True)
            p = np.exp(z)
            p = p / p.sum(axis=1, keepdims=True)
            out[sel, h, :] = p @ v[a:a + nk, c, :]
    return out


def softplus(x: np.ndarray) -> np.ndarray:
    """log(1 + e^x), evaluated as max(x, 0) + log1p(e^-|x|) (no overflow)."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def query_temperature(sigma: np.ndarray, positions: np.ndarray, kept_offsets: Sequence[int]) -> np.ndarray:
    """Per-query temperature of the kept rows ([reading] §4.1, component two,
    second refinement): pruning shrinks the keys a query sees from its
    original position p_i to its rank m_i among the kept tokens, which
    sharpens the softmax; the temperature
        tau_ih = softplus(sigma_h) * log(m_i) / log(max(2, p_i))
    recalibrates it.  Readings: p_i = 1 + the row's original 0-based position
    inside its prompt (the number of keys it sees unpruned) and m_i = 1 + its
    0-based kept row inside the prompt (the number of kept keys it sees);
    sigma is one value per (layer, head).  With nothing pruned m_i = p_i and
    the factor is 1 (0 for the first row, whose single key makes any
    temperature equivalent).

    sigma [Hq]; positions [M] int (original positions of the kept rows, in
    kept order); returns tau [M, Hq] float64.
    Pinned by the no-pruning reduction, a two-key closed form and the
    vanishing-temperature limit (tests/test_oracle_attention.py).
    """
    sigma = np.asarray(sigma, dtype=np.float64)
    positions = np.asarray(positions, dtype=np.int64)
    offs = [int(o) for o in kept_offsets]
    m_rank = np.zeros(positions.size, dtype=np.float64)
    for a, b in zip(offs[:-1], offs[1:]):
        m_rank[a:b] = np.arange(1, b - a + 1)
    p = np.maximum(2.0, positions.astype(np.float64) + 1.0)
    return softplus(sigma)[None, :] * (np.log(m_rank) / np.log(p))[:, None]


def gated_attention_decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, s: Optional[np.ndarray],
                           tau: Optional[np.ndarray], gain: Optional[np.ndarray], lens: Sequence[int]) -> np.ndarray:
    """One decode step of token-gated attention over a pruned KV cache
    ([reading] §4.1 component one: pruned tokens leave no KV entry and the
    tokens being decoded are not prunable, score 0; engineering notes: at
    decode time the gate term becomes an additive attention mask).

    Sequence b's new query q[b] (its own K/V already appended) attends to the
    cache rows j < lens[b]:
        z_j = tau_h (q_h . k_j) / sqrt(D) + g_h s_j,   out[b, h] = sum_j softmax_j(z) v_j
    i.e. the additive mask is g_h s_j.  q [B, Hq, D]; k_cache / v_cache
    [B, cap, Hkv, D]; s [B, cap] (0 for generated or question tokens) or None;
    tau [Hq], [B, Hq] (a temperature per query) or None (= 1); gain [Hq] or
    None.  An empty cache (lens[b] = 0) gives a zero output.
    Pinned by row-by-row equality with the prefill oracle (causal attention is
    decode applied to every prefix), a two-key closed form and the empty and
    single-key cases.
    """
    q = np.asarray(q, dtype=np.float64)
    k_cache = np.asarray(k_cache, dtype=np.float64)
    v_cache = np.asarray(v_cache, dtype=np.float64)
    bsz, hq, dh = q.shape
    hkv = k_cache.shape[2]
    group = hq // hkv
    tau = np.ones(hq) if tau is None else np.asarray(tau, dtype=np.float64)
    if tau.ndim == 1:
        tau = np.broadcast_to(tau[None, :], (bsz, hq))
    use_bias = s is not None and gain is not None
    out = np.zeros((bsz, hq, dh), dtype=np.float64)
    for b in range(bsz):
        n = int(lens[b])
        if n == 0:
            continue
        for h in range(hq):
            c = h // group
            z = tau[b, h] * (k_cache[b, :n, c, :] @ q[b, h, :]) / math.sqrt(dh)
            if use_bias:
                z = z + float(gain[h]) * np.asarray(s[b, :n], dtype=np.float64)
            p = np.exp(z - z.max())
            out[b, h, :] = (p / p.sum()) @ v_cache[b, :n, c, :]
    return out


def gated_attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, s: Optional[np.ndarray],
                             tau: Optional[np.ndarray], gain: Optional[np.ndarray], kept_offsets: Sequence[int],
                             dout: np.ndarray) -> dict:
    """Gradients of the token-gated attention (the forward of gated_attention)
    with respect to q, k, v, the key scores s, the gains g_h and the
    temperatures tau_h, for an upstream gradient dout [M, Hq, D]
    ([reading] §4.1 engineering notes: the same attention kernel accumulates
    the bias gradient back into the scorer in the backward pass).

    Per prompt and head, with z = tau q.k/sqrt(D) + g s (causal), P = softmax(z):
        dV   = P^T dO                       (summed over the heads sharing a KV head)
        dZ   = P o (dO V^T - rowsum(dO o O))
        dQ   = tau/sqrt(D) dZ K,   dK = tau/sqrt(D) dZ^T Q  (dK summed like dV)
        ds_t = sum_h g_h sum_r dZ_rt,   dg_h = sum_rt dZ_rt s_t,   dtau_h = sum_rt dZ_rt q_r.k_t/sqrt(D)
    Returns a dict of float64 arrays: dq [M, Hq, D], dk, dv [M, Hkv, D],
    ds [M], dgain [Hq], dtau [Hq] (the last three zero without a bias / with
    tau None, where they are not inputs).
    Pinned by central finite differences of gated_attention and by torch
    autograd on the same forward (tests/test_oracle_attention.py).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    m_total, hq, dh = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    tau_v = np.ones(hq) if tau is None else np.asarray(tau, dtype=np.float64)
    use_bias = s is not None and gain is not None
    s_v = np.asarray(s, dtype=np.float64) if use_bias else np.zeros(m_total)
    g_v = np.asarray(gain, dtype=np.float64) if use_bias else np.zeros(hq)
    scale = 1.0 / math.sqrt(dh)
    res = {"dq": np.zeros_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v), "ds": np.zeros(m_total),
           "dgain": np.zeros(hq), "dtau": np.zeros(hq)}
    offs = [int(o) for o in kept_offsets]
    for a, b in zip(offs[:-1], offs[1:]):
        n = b - a
        if n == 0:
            continue
        causal = np.tril(np.ones((n, n), dtype=bool))
        for h in range(hq):
            c = h // group
            qh, kc, vc, do = q[a:b, h], k[a:b, c], v[a:b, c], dout[a:b, h]
            qk = (qh @ kc.T) * scale
            z = np.where(causal, tau_v[h] * qk + g_v[h] * s_v[a:b][None, :], -np.inf)
            z = z - z.max(axis=1, keepdims=True)
            p = np.exp(z)
            p = p / p.sum(axis=1, keepdims=True)
            o = p @ vc
            dp = do @ vc.T
            dz = p * (dp - (do * o).sum(axis=1, keepdims=True))
            res["dv"][a:b, c] += p.T @ do
            res["dq"][a:b, h] += tau_v[h] * scale * (dz @ kc)
            res["dk"][a:b, c] += tau_v[h] * scale * (dz.T @ qh)
            res["ds"][a:b] += g_v[h] * dz.sum(axis=0)
            res["dgain"][h] += (dz.sum(axis=0) * s_v[a:b]).sum()
            res["dtau"][h] += (dz * qk).sum()
    return res


def attention_logsumexp(q: np.ndarray, k: np.ndarray, s: Optional[np.ndarray], tau: Optional[np.ndarray],
                        gain: Optional[np.ndarray], kept_offsets: Sequence[int]) -> np.ndarray:
    """ln sum_{t <= r} exp(z_rt) for every kept row r and query head h, with
    the logits of gated_attention: the normaliser of the row's softmax, which
    a flash-style backward keeps from the forward.  Returns [M, Hq] float64.
    Pinned by the uniform-logit closed form ln(r + 1) and by the weights
    exp(z - lse) summing to 1 (tests/test_oracle_attention.py)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    m_total, hq, dh = q.shape
    group = hq // k.shape[1]
    tau = np.ones(hq) if tau is None else np.asarray(tau, dtype=np.float64)
    use_bias = s is not None and gain is not None
    out = np.zeros((m_total, hq))
    offs = [int(o) for o in kept_offsets]
    for a, b in zip(offs[:-1], offs[1:]):
        n = b - a
        if n == 0:
            continue
        causal = np.tril(np.ones((n, n), dtype=bool))
        for h in range(hq):
            z = tau[h] * (q[a:b, h] @ k[a:b, h // group].T) / math.sqrt(dh)
            if use_bias:
                z = z + float(gain[h]) * np.asarray(s[a:b], dtype=np.float64)[None, :]
            z = np.where(causal, z, -np.inf)
            mx = z.max(axis=1)
            out[a:b, h] = mx + np.log(np.exp(z - mx[:, None]).sum(axis=1))
    return out
