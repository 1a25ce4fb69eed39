"""Reference (float64, CPU) of the pruned-prefill decoder stack -- TEST
INFRASTRUCTURE (see the package docstring).

TokenGate's forward ([reading] §4.1, three-stage forward): layers 0 .. L-1
process every token; at layer L the gate scores the document tokens from the
normalised post-attention residual; the layers above process only the kept
tokens with token-gated attention and create no KV entries for pruned tokens.
The layer itself is a Qwen3-shaped pre-norm decoder layer (RMSNorm, GQA
attention with rotary embedding, SwiGLU MLP, residual adds).  Readings used
here, not stated on the pages: rotate-half rotary embedding at the original
token positions (also above the gate), theta = 1e6; the gate reads layer L's
RMSNorm(h) (the MLP input) and the kept rows of layer L's output residual
continue to layer L + 1.

"bf16 throughout" is modelled by rounding every tensor that the layer stores
between two steps to bf16 (round to nearest even), computing each step in
float64.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence

import numpy as np

from .tokengate_ref import gate_scores, gated_attention, kept_indices


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (8 significant bits, ties to even), as float64.
    Written here from the definition of the format (sign, 8-bit exponent,
    7 stored mantissa bits); NaN and inf pass through."""
    a = np.asarray(a, dtype=np.float64)
    f = a.astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    out = rounded.astype(np.uint32).view(np.float32).astype(np.float64)
    special = ~np.isfinite(a)
    if special.any():
        out = np.where(special, a, out)
    return out


def rmsnorm(x: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * weight, per row."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(weight, dtype=np.float64)


def rope(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half rotary embedding of x [m, heads, D] at integer positions:
    pair (i, i + D/2) is rotated by angle p * theta^(-2 i / D)."""
    x = np.asarray(x, dtype=np.float64)
    dh = x.shape[-1]
    half = dh // 2
    inv = theta ** (-2.0 * np.arange(half) / dh)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(v: np.ndarray) -> np.ndarray:
    return v / (1.0 + np.exp(-v))


class LayerWeights:
    """Weights of one layer as float64 arrays (bf16-valued).  w_gate and w_up
    are separate here; the GPU layout interleaves them."""

    def __init__(self, attn_norm, wq, wk, wv, wo, mlp_norm, w_gate, w_up, w_down, tau=None, gain=None):
        self.attn_norm, self.wq, self.wk, self.wv, self.wo = attn_norm, wq, wk, wv, wo
        self.mlp_norm, self.w_gate, self.w_up, self.w_down = mlp_norm, w_gate, w_up, w_down
        self.tau, self.gain = tau, gain


def decoder_layer(x: np.ndarray, positions: np.ndarray, key_score: Optional[np.ndarray], w: LayerWeights,
                  kept_offsets: Sequence[int], hq: int, hkv: int, dh: int, eps: float, theta: float,
                  bf16: bool = True):
    """One pre-norm decoder layer over the rows x [m, d] (prompts given by
    kept_offsets), causal within each prompt.  Returns (y, rmsnorm(h)).
    key_score (the kept rows' gate scores) with w.gain turns the attention into
    token-gated attention; w.tau scales q.k."""
    r = round_bf16 if bf16 else (lambda a: np.asarray(a, dtype=np.float64))
    m = x.shape[0]
    xn = r(rmsnorm(x, w.attn_norm, eps))
    q = r(xn @ w.wq.T).reshape(m, hq, dh)
    k = r(xn @ w.wk.T).reshape(m, hkv, dh)
    v = r(xn @ w.wv.T).reshape(m, hkv, dh)
    q = r(rope(q, positions, theta))
    k = r(rope(k, positions, theta))
    a = gated_attention(q, k, v, key_score if w.gain is not None else None, w.tau, w.gain, kept_offsets)
    a = r(a).reshape(m, hq * dh)
    h = r(x + a @ w.wo.T)
    hn = r(rmsnorm(h, w.mlp_norm, eps))
    mid = r(silu(hn @ w.w_gate.T) * (hn @ w.w_up.T))
    y = r(h + mid @ w.w_down.T)
    return y, hn


def pruned_stack(x0: np.ndarray, layers: List[LayerWeights], gate_layer: int, gate_w1: np.ndarray,
                 gate_w2: np.ndarray, seg_start: Sequence[int], doc_begin: Sequence[int], doc_end: Sequence[int],
                 k_budget: Sequence[int], hq: int, hkv: int, dh: int, eps: float = 1e-6, theta: float = 1e6,
                 gate_eps: float = 1e-6, bf16: bool = True, kept_idx: Optional[np.ndarray] = None):
    """Layers 0 .. gate_layer over every token; the gate on layer
    gate_layer's RMSNorm(h); top-K select; layers above over the kept rows
    (original positions, gated attention).  Returns (y_kept, kept_idx,
    kept_offsets, scores).  kept_idx, when given, replaces the select's
    result (a test that must follow another selector's choice at a near-tie
    of the scores passes it; the offsets are those of the budgets)."""
    n = x0.shape[0]
    pos = np.arange(n)
    full_offs = list(seg_start)
    for i in range(len(seg_start) - 1):  # positions restart in every prompt
        pos[seg_start[i]:seg_start[i + 1]] -= seg_start[i]
    x = np.asarray(x0, dtype=np.float64)
    hn = None
    for li in range(gate_layer + 1):
        x, hn = decoder_layer(x, pos, None, layers[li], full_offs, hq, hkv, dh, eps, theta, bf16)
    s = gate_scores(hn, gate_w1, None, gate_w2, 0.0, seg_start, doc_begin, doc_end, gate_eps)
    if bf16:
        s = s.astype(np.float32).astype(np.float64)  # the scores are stored as fp32
    idx, offs = kept_indices(s, seg_start, doc_begin, doc_end, k_budget)
    if kept_idx is not None:
        kept_idx = np.asarray(kept_idx, dtype=np.int64)
        assert kept_idx.shape == idx.shape, "a kept set of the budgets' size"
        idx = kept_idx
    xk, pk, sk = x[idx], pos[idx], s[idx]
    for li in range(gate_layer + 1, len(layers)):
        xk, _ = decoder_layer(xk, pk, sk, layers[li], offs, hq, hkv, dh, eps, theta, bf16)
    return xk, idx, offs, s
