"""Seeded synthetic inputs for the TokenGate pruned-prefill path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic, so both the CPU oracle (through the tests) and the HIP
path can consume exactly the same arrays.

The workloads stand in for the needle-in-a-haystack prompts the TokenGate
write-ups time at 16K-128K tokens (a document followed by a short question,
one prunable document span per prompt).  A handful of planted "needle" rows
with a larger norm play the role of the single retrieval target.

Recipe (per workload): ``numpy.random.Generator(PCG64(seed))``; draws happen
in a fixed order, in float32, then bf16 tensors are rounded to nearest-even
on the host.  bf16 tensors are carried as ``uint16`` bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

# ----------------------------------------------------------------------------
# bf16 helpers (bit manipulation only)
# ----------------------------------------------------------------------------


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); returns uint16 bits.

    NaN stays NaN (quiet bit forced); infinities stay infinities.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    lsb = (u >> 16) & 1
    r = ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)
    if nan.any():
        r = np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), r)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


# ----------------------------------------------------------------------------
# Segment layout
# ----------------------------------------------------------------------------


@dataclass
class Segments:
    """Packed batch of prompts.  Token t of segment i lives at seg_start[i] + t.

    doc_begin / doc_end are relative to the segment; every token outside
    [doc_begin, doc_end) is non-prunable (instruction / question).
    """

    seg_start: List[int]
    doc_begin: List[int]
    doc_end: List[int]
    k_budget: List[int]

    @property
    def n_seg(self) -> int:
        return len(self.doc_begin)

    @property
    def n_tokens(self) -> int:
        return self.seg_start[-1]

    def seg_len(self, i: int) -> int:
        return self.seg_start[i + 1] - self.seg_start[i]

    def n_doc(self, i: int) -> int:
        return self.doc_end[i] - self.doc_begin[i]

    def with_budget(self, k) -> "Segments":
        if isinstance(k, int):
            k = [k] * self.n_seg
        return Segments(list(self.seg_start), list(self.doc_begin), list(self.doc_end), list(k))


def single_segment(n_doc: int, n_q: int, k: int) -> Segments:
    """One prompt: document first, question last."""
    return Segments([0, n_doc + n_q], [0], [n_doc], [k])


def random_segments(rng: np.random.Generator, n_seg: int, max_len: int, min_len: int = 1) -> Segments:
    """Several prompts of ragged length, each with a random document span
    (possibly empty, possibly the whole prompt) and a random budget that may
    exceed the document (clamped by the method) or be zero."""
    lens = rng.integers(min_len, max_len + 1, size=n_seg)
    seg_start = [0]
    doc_begin, doc_end, kb = [], [], []
    for L in lens:
        L = int(L)
        seg_start.append(seg_start[-1] + L)
        a = int(rng.integers(0, L + 1))
        b = int(rng.integers(a, L + 1))
        doc_begin.append(a)
        doc_end.append(b)
        kb.append(int(rng.integers(0, (b - a) + 3)))
    return Segments(seg_start, doc_begin, doc_end, kb)


# ----------------------------------------------------------------------------
# Gated-layer workloads
# ----------------------------------------------------------------------------


@dataclass
class GatedLayer:
    name: str
    segments: Segments
    d: int
    h: int
    hq: int
    hkv: int
    head_dim: int
    x: np.ndarray  # uint16 bf16 [N, d]  hidden rows the gate reads (also the rows compacted)
    w1: np.ndarray  # uint16 bf16 [h, d]
    b1: np.ndarray  # float32 [h]
    w2: np.ndarray  # float32 [h]
    b2: float
    q: Optional[np.ndarray] = None  # uint16 bf16 [N, hq, D]
    k: Optional[np.ndarray] = None  # uint16 bf16 [N, hkv, D]
    v: Optional[np.ndarray] = None  # uint16 bf16 [N, hkv, D]
    gain: Optional[np.ndarray] = None  # float32 [hq]
    tau: Optional[np.ndarray] = None  # float32 [hq]
    needle_rows: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))
    k_sweep: Sequence[int] = ()


def _xavier(rng, fan_out, fan_in, size):
    std = np.sqrt(2.0 / (fan_in + fan_out))
    return (rng.standard_normal(size, dtype=np.float32) * np.float32(std)).astype(np.float32)


def make_gated_layer(
    seed: int,
    segments: Segments,
    d: int,
    h: int,
    hq: int,
    hkv: int,
    head_dim: int,
    n_needles: int = 0,
    needle_scale: float = 1.0,
    with_qkv: bool = True,
    name: str = "custom",
) -> GatedLayer:
    """Draw order: X, needle rows, W1, w2, Q, K, V, gain, tau.  Biases are 0."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n = segments.n_tokens
    x = rng.standard_normal((n, d), dtype=np.float32)
    doc_rows = np.concatenate(
        [np.arange(segments.seg_start[i] + segments.doc_begin[i], segments.seg_start[i] + segments.doc_end[i])
         for i in range(segments.n_seg)] + [np.zeros(0, np.int64)]
    ).astype(np.int64)
    needles = np.zeros(0, np.int64)
    if n_needles > 0 and doc_rows.size > 0:
        needles = np.sort(rng.choice(doc_rows, size=min(n_needles, doc_rows.size), replace=False))
        x[needles] *= np.float32(needle_scale)
    w1 = _xavier(rng, h, d, (h, d))
    w2 = _xavier(rng, 1, h, (h,))
    layer = GatedLayer(
        name=name, segments=segments, d=d, h=h, hq=hq, hkv=hkv, head_dim=head_dim,
        x=f32_to_bf16_bits(x), w1=f32_to_bf16_bits(w1),
        b1=np.zeros(h, np.float32), w2=w2.astype(np.float32), b2=0.0,
        needle_rows=needles,
    )
    del x
    if with_qkv:
        layer.q = f32_to_bf16_bits(rng.standard_normal((n, hq, head_dim), dtype=np.float32))
        layer.k = f32_to_bf16_bits(rng.standard_normal((n, hkv, head_dim), dtype=np.float32))
        layer.v = f32_to_bf16_bits(rng.standard_normal((n, hkv, head_dim), dtype=np.float32))
        layer.gain = rng.uniform(0.5, 1.5, size=hq).astype(np.float32)
        layer.tau = rng.uniform(0.8, 1.2, size=hq).astype(np.float32)
    return layer


def mixture_scores(seed: int, segments: Segments, k_marks: Sequence[int] = (), n_signed_zero: int = 8) -> np.ndarray:
    """fp32 select input: doc positions draw 95 % N(0,1) and 5 % N(4, 0.5);
    1 % of doc positions are then overwritten with exact copies of other
    positions' values.  For every budget in ``k_marks`` a group of six equal
    values is planted across the budget boundary (ranks K-3 .. K+2), and a few
    +0.0 / -0.0 values are planted.  Non-doc positions hold unrelated values
    (the selector must ignore them).  Order of draws is fixed."""
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    n = segments.n_tokens
    s = rng.standard_normal(n, dtype=np.float32)
    for i in range(segments.n_seg):
        lo = segments.seg_start[i] + segments.doc_begin[i]
        hi = segments.seg_start[i] + segments.doc_end[i]
        nd = hi - lo
        if nd == 0:
            continue
        hot = rng.random(nd) < 0.05
        vals = np.where(hot, rng.normal(4.0, 0.5, nd), rng.standard_normal(nd)).astype(np.float32)
        n_dup = max(1, nd // 100)
        dst = rng.choice(nd, size=n_dup, replace=False)
        src = rng.integers(0, nd, size=n_dup)
        vals[dst] = vals[src]
        order = np.argsort(-vals.astype(np.float64), kind="stable")
        for k in k_marks:
            if 3 <= k <= nd - 3:
                grp = order[k - 3:k + 3]
                vals[grp] = vals[order[k - 1]]
        if n_signed_zero > 0 and nd >= 2 * n_signed_zero:
            z = rng.choice(nd, size=n_signed_zero, replace=False)
            vals[z[: n_signed_zero // 2]] = np.float32(0.0)
            vals[z[n_signed_zero // 2:]] = np.float32(-0.0)
        s[lo:hi] = vals
    return s


# ----------------------------------------------------------------------------
# The five workloads
# ----------------------------------------------------------------------------

WORKLOADS = {
    1: dict(name="tiny-gated-layer N=512 d=256 K=128", n_doc=448, n_q=64, d=256, h=64, hq=4, hkv=2, D=64,
            k=128, needles=8, needle_scale=4.0),
    2: dict(name="gated-layer N=16384 d=2048 K=2048", n_doc=16320, n_q=64, d=2048, h=256, hq=16, hkv=8, D=128,
            k=2048, needles=32, needle_scale=3.0),
    3: dict(name="gated-layer N=32768 d=2048 K-sweep", n_doc=32704, n_q=64, d=2048, h=256, hq=16, hkv=8, D=128,
            k=2048, needles=32, needle_scale=3.0, k_sweep=(1024, 2048, 4096, 8192)),
    4: dict(name="gated-layer N=131072 d=2048 K=4096", n_doc=131008, n_q=64, d=2048, h=256, hq=16, hkv=8, D=128,
            k=4096, needles=32, needle_scale=3.0, k_sweep=(2048, 4096)),
}


def workload(index: int, k: Optional[int] = None, with_qkv: bool = True) -> GatedLayer:
    """Workload ``index`` (1-4) with seed = index."""
    w = WORKLOADS[index]
    seg = single_segment(w["n_doc"], w["n_q"], w["k"] if k is None else k)
    layer = make_gated_layer(index, seg, w["d"], w["h"], w["hq"], w["hkv"], w["D"],
                             n_needles=w["needles"], needle_scale=w["needle_scale"], with_qkv=with_qkv,
                             name=w["name"])
    layer.k_sweep = w.get("k_sweep", (seg.k_budget[0],))
    return layer
