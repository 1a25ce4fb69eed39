"""Pruned-prefill decoder stack on the HIP library.

Layers 0 .. gate_layer run over every token; the gate scores the documents
from gate_layer's normalised post-attention residual; the top-K selector and
the compaction keep the best document rows plus every non-document row; the
remaining layers run only on the kept rows, with token-gated attention and
rotary embedding at the original positions ("TokenGate 与 T2Quant ... 精读",
section 4.1, three-stage forward).  Every step is a libtokengate call; this
module only sequences them and owns the device buffers.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

from . import tokengate as tg


def interleave_gate_up(w_gate: torch.Tensor, w_up: torch.Tensor) -> torch.Tensor:
    """[f, d] gate and up rows -> [2f, d] in groups of 8 (gate 8j..8j+7, up 8j..8j+7), the SwiGLU GEMM layout."""
    f, d = w_gate.shape
    return torch.stack([w_gate.reshape(f // 8, 8, d), w_up.reshape(f // 8, 8, d)], dim=1).reshape(2 * f, d).contiguous()


@dataclass
class DeviceLayer:
    attn_norm: torch.Tensor
    wqkv: torch.Tensor
    wo: torch.Tensor
    mlp_norm: torch.Tensor
    w_gate_up: torch.Tensor
    w_down: torch.Tensor
    tau: Optional[torch.Tensor] = None
    gain: Optional[torch.Tensor] = None
    c_struct: tg.LayerWeights = field(init=False)

    def __post_init__(self):
        p = lambda t: None if t is None else t.data_ptr()
        self.c_struct = tg.LayerWeights(p(self.attn_norm), p(self.wqkv), p(self.wo), p(self.mlp_norm),
                                        p(self.w_gate_up), p(self.w_down), p(self.tau), p(self.gain))


def random_layers(seed: int, n_layers: int, gated_from: int, d: int, hq: int, hkv: int, dh: int, f: int,
                  device, std: float = 0.02) -> List[DeviceLayer]:
    """Seeded random-init layers drawn on the device: weights N(0, std^2) in
    bf16, RMSNorm weights 1, and for layers >= gated_from a temperature
    U(0.8, 1.2) and gate gain U(0.5, 1.5) per head."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = []
    nqkv = (hq + 2 * hkv) * dh

    def normal(*shape):
        return (torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std).to(torch.bfloat16)

    for li in range(n_layers):
        gated = li >= gated_from
        tau = (0.8 + 0.4 * torch.rand(hq, generator=gen, device=device)) if gated else None
        gain = (0.5 + torch.rand(hq, generator=gen, device=device)) if gated else None
        out.append(DeviceLayer(torch.ones(d, dtype=torch.bfloat16, device=device), normal(nqkv, d),
                               normal(d, hq * dh), torch.ones(d, dtype=torch.bfloat16, device=device),
                               normal(2 * f, d), normal(d, f), tau, gain))
    return out


def positions_of(plan: tg.Plan) -> np.ndarray:
    """Position of every token inside its prompt (restarting at 0 per prompt)."""
    pos = np.zeros(plan.n_tokens, dtype=np.int32)
    for s0, ln in plan.table[:, :2]:
        pos[s0:s0 + ln] = np.arange(ln, dtype=np.int32)
    return pos


@dataclass
class StackPlan:
    """Host-built segment tables of one batch: `full` covers every token (each
    document kept whole), `pruned` applies the budgets; `pos` holds the
    in-prompt positions on the device."""
    full: tg.Plan
    pruned: tg.Plan
    pos: torch.Tensor


class PrunedStack:
    def __init__(self, layers: List[DeviceLayer], gate_layer: int, gate_w1: torch.Tensor, gate_w2: torch.Tensor,
                 d: int, hq: int, hkv: int, dh: int, f: int, eps: float = 1e-6, theta: float = 1e6,
                 gate_eps: float = 1e-6):
        self.layers, self.gate_layer = layers, gate_layer
        self.gate_w1, self.gate_w2 = gate_w1, gate_w2
        self.d, self.hq, self.hkv, self.dh, self.f = d, hq, hkv, dh, f
        self.eps, self.theta, self.gate_eps = eps, theta, gate_eps
        self._ws = None
        self.gate_w1_packed = tg.gate_pack_w1(gate_w1)  # fragment order, packed once

    def plan(self, seg_start, doc_begin, doc_end, k_budget, device) -> StackPlan:
        full = tg.plan_segments(seg_start, doc_begin, doc_end, [e - b for b, e in zip(doc_begin, doc_end)], device)
        pruned = tg.plan_segments(seg_start, doc_begin, doc_end, k_budget, device)
        return StackPlan(full, pruned, torch.from_numpy(positions_of(full)).to(device))

    def _workspace(self, rows, device):
        need = max(tg.decoder_layer_workspace_bytes(rows, self.d, self.hq, self.hkv, self.dh, self.f), 256)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=device)
        return self._ws

    def _layer(self, li, hidden, pos, score, plan, ws, post=None):
        tg.decoder_layer(hidden, pos, score, plan, self.layers[li].c_struct, self.d, self.hq, self.hkv, self.dh,
                         self.f, ws, self.eps, self.theta, post)

    def buffers(self, x: torch.Tensor, plan: StackPlan, prune: bool = True) -> dict:
        """Every buffer one forward over this batch layout uses (hidden rows, gate input, scores, kept indices,
        compacted rows, positions and scores, and the workspaces), allocated once: a forward given them
        allocates nothing, so it can be captured as a graph.  A captured graph keeps its own set (the layer
        workspace shared by eager forwards may be reallocated later)."""
        dev = x.device
        n, m = plan.full.total_kept, plan.pruned.total_kept
        h = self.gate_w1.shape[0]
        b = {"hidden": torch.empty_like(x), "gate_in": torch.empty_like(x)}
        b["layer_ws"] = torch.empty(max(tg.decoder_layer_workspace_bytes(n, self.d, self.hq, self.hkv, self.dh,
                                                                         self.f), 256), dtype=torch.uint8, device=dev)
        if prune:
            b["scores"] = torch.empty(n, dtype=torch.float32, device=dev)
            b["kept"] = torch.empty(m, dtype=torch.int32, device=dev)
            b["hk"] = torch.empty((m, self.d), dtype=torch.bfloat16, device=dev)
            b["pk"] = torch.empty(m, dtype=torch.int32, device=dev)
            b["sk"] = torch.empty(m, dtype=torch.float32, device=dev)
            b["gate_ws"] = torch.empty(max(tg.gate_workspace_bytes(plan.pruned, self.d, h), 256), dtype=torch.uint8,
                                       device=dev)
            b["select_ws"] = torch.empty(max(tg.select_workspace_bytes(plan.pruned), 256), dtype=torch.uint8,
                                         device=dev)
        return b

    def _eager_buffers(self, x: torch.Tensor, plan: StackPlan, prune: bool) -> dict:
        """Fresh output buffers; the layer workspace is kept between eager calls and grown when needed."""
        n, m = plan.full.total_kept, plan.pruned.total_kept
        dev = x.device
        b = {"hidden": torch.empty_like(x), "gate_in": torch.empty_like(x), "layer_ws": self._workspace(n, dev)}
        if prune:
            h = self.gate_w1.shape[0]
            b.update(scores=torch.empty(n, dtype=torch.float32, device=dev),
                     kept=torch.empty(m, dtype=torch.int32, device=dev),
                     hk=torch.empty((m, self.d), dtype=torch.bfloat16, device=dev),
                     pk=torch.empty(m, dtype=torch.int32, device=dev),
                     sk=torch.empty(m, dtype=torch.float32, device=dev),
                     gate_ws=tg._workspace(tg.gate_workspace_bytes(plan.pruned, self.d, h), dev),
                     select_ws=tg._workspace(tg.select_workspace_bytes(plan.pruned), dev))
        return b

    def forward(self, x: torch.Tensor, seg_start=None, doc_begin=None, doc_end=None, k_budget=None,
                prune: bool = True, plan: Optional[StackPlan] = None, mark=None, bufs: Optional[dict] = None) -> dict:
        """x bf16 [N, d] (not modified).  prune=False runs every layer over
        every token.  `plan` (from plan()) saves rebuilding the tables;
        `mark(name)`, if given, is called on the host after the launches of
        each phase ("lower", "prune", "upper") have been issued.  `bufs` (from
        buffers()) makes the forward allocate nothing."""
        dev = x.device
        if plan is None:
            plan = self.plan(seg_start, doc_begin, doc_end, k_budget, dev)
        if bufs is None:
            bufs = self._eager_buffers(x, plan, prune)
        full, pos, ws = plan.full, plan.pos, bufs["layer_ws"]
        hidden, gate_in = bufs["hidden"], bufs["gate_in"]
        hidden.copy_(x)
        for li in range(self.gate_layer + 1):
            self._layer(li, hidden, pos, None, full, ws, gate_in if li == self.gate_layer else None)
        if mark:
            mark("lower")
        if not prune:
            for li in range(self.gate_layer + 1, len(self.layers)):
                self._layer(li, hidden, pos, None, full, ws)
            if mark:
                mark("upper")
            return {"hidden": hidden, "gate_in": gate_in}
        pp = plan.pruned
        scores, kept, hk, pk, sk = bufs["scores"], bufs["kept"], bufs["hk"], bufs["pk"], bufs["sk"]
        tg.gate_score_prepacked(gate_in, self.gate_w1_packed, self.gate_w1.shape[0], None, self.gate_w2, 0.0, pp,
                                rms_eps=self.gate_eps, scores=scores, workspace=bufs["gate_ws"])
        tg.select_topk(scores, pp, kept_idx=kept, workspace=bufs["select_ws"])
        tg.compact_kept(kept, [(hidden, hk), (pos, pk), (scores, sk)])
        if mark:
            mark("prune")
        for li in range(self.gate_layer + 1, len(self.layers)):
            self._layer(li, hk, pk, sk, pp, ws)
        if mark:
            mark("upper")
        return {"hidden": hk, "kept": kept, "scores": scores, "plan": pp, "gate_in": gate_in}

    def capture(self, x: torch.Tensor, plan: StackPlan, prune: bool = True) -> "StackGraph":
        """The whole forward over this batch layout (lower layers, gate, select, compaction, upper layers) as one
        HIP graph: the pages capture the pruned forward as a graph per padded length; here the kept count is
        known on the host from the budgets, so one graph per layout needs no padding.  Nothing in it allocates,
        synchronises or memsets (the select's counters are cleared by a kernel)."""
        bufs = self.buffers(x, plan, prune)
        side = torch.cuda.Stream(device=x.device)
        side.wait_stream(torch.cuda.current_stream(x.device))
        with torch.cuda.stream(side):  # warm the stream (and the library's lazily cached state) before capture
            out = self.forward(x, plan=plan, prune=prune, bufs=bufs)
        torch.cuda.current_stream(x.device).wait_stream(side)
        torch.cuda.synchronize(x.device)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            out = self.forward(x, plan=plan, prune=prune, bufs=bufs)
        torch.cuda.synchronize(x.device)
        return StackGraph(g, out, bufs)


@dataclass
class StackGraph:
    """A captured forward: replay() runs it again on the input it was captured with (x's storage) and leaves
    the results in `out` (the buffers of the capture)."""
    graph: "torch.cuda.CUDAGraph"
    out: dict
    bufs: dict

    def replay(self) -> dict:
        self.graph.replay()
        return self.out
