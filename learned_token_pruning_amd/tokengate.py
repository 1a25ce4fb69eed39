"""Python binding of libtokengate (ctypes).

Argument marshalling only: every step of the path runs in the HIP kernels of
``libtokengate.so``.  torch provides device memory and streams.  Importing
this module loads the library and raises ImportError when it has not been
built (``python -m learned_token_pruning_amd.build``); there is no other code
path.

The names mirror the C ABI in include/tokengate.h: plan_segments,
gate_score, select_topk, compact_kept, gated_attention_prefill.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch  # loads the HIP runtime first, so the library binds to the same one

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtokengate.so")

if not os.path.exists(_LIB_PATH):
    raise ImportError(f"libtokengate.so is not built ({_LIB_PATH}); run `python -m learned_token_pruning_amd.build`")

_lib = ctypes.CDLL(_LIB_PATH, mode=ctypes.RTLD_GLOBAL)

TG_OK = 0
STATUS_NAMES = {0: "TG_OK", -1: "TG_ERR_INVALID_ARG", -2: "TG_ERR_UNSUPPORTED", -3: "TG_ERR_WORKSPACE",
                -4: "TG_ERR_NO_DEVICE", -5: "TG_ERR_HIP"}
EXPORTS = ("tg_status_string", "tg_abi_version", "tg_plan_segments", "tg_kept_count", "tg_gate_workspace_bytes",
           "tg_gate_score", "tg_gate_packed_w1_bytes", "tg_gate_pack_w1", "tg_gate_score_prepacked",
           "tg_gate_score_prepacked_noalloc", "tg_gate_noalloc_max_tiles",
           "tg_select_workspace_bytes", "tg_select_topk", "tg_compact_kept", "tg_gated_attention_prefill",
           "tg_attention_prefill_workspace_bytes", "tg_gated_attention_prefill_ws", "tg_attention_workspace_status",
           "tg_gated_attention_prefill_gather_ws", "tg_gated_attention_prefill_query_tau_ws",
           "tg_gated_attention_prefill_gather", "tg_gated_attention_prefill_query_tau",
           "tg_decode_workspace_bytes", "tg_gated_attention_decode", "tg_gated_attention_prefill_lse",
           "tg_attention_backward_workspace_bytes", "tg_gated_attention_backward",
           "tg_gemm_bf16", "tg_rmsnorm_bf16", "tg_rope_split_bf16", "tg_decoder_layer_workspace_bytes",
           "tg_decoder_layer")
GEMM_STORE, GEMM_RESIDUAL, GEMM_SWIGLU = 0, 1, 2
COMPACT_MAX_TENSORS = 8


class TokenGateError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({status_string(status)})")


class Segment(ctypes.Structure):
    _fields_ = [("seg_start", ctypes.c_int32), ("seg_len", ctypes.c_int32), ("doc_begin", ctypes.c_int32),
                ("doc_end", ctypes.c_int32), ("k_eff", ctypes.c_int32), ("kept_start", ctypes.c_int32),
                ("kept_len", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int64), ("total_kept", ctypes.c_int64), ("n_seg", ctypes.c_int32),
                ("max_seg_len", ctypes.c_int32), ("max_doc_len", ctypes.c_int32), ("max_kept_len", ctypes.c_int32)]


class LayerWeights(ctypes.Structure):
    _fields_ = [("attn_norm", ctypes.c_void_p), ("wqkv", ctypes.c_void_p), ("wo", ctypes.c_void_p),
                ("mlp_norm", ctypes.c_void_p), ("w_gate_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("tau", ctypes.c_void_p), ("gain", ctypes.c_void_p)]


_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int
_f32 = ctypes.c_float
_sz = ctypes.c_size_t

_lib.tg_status_string.restype = ctypes.c_char_p
_lib.tg_status_string.argtypes = [_i32]
_lib.tg_abi_version.restype = _i32
_lib.tg_kept_count.restype = _i64
_lib.tg_kept_count.argtypes = [_i64, _i64, _i64]
_lib.tg_plan_segments.restype = _i32
_lib.tg_plan_segments.argtypes = [_i32, _vp, _vp, _vp, _vp, ctypes.POINTER(Segment), ctypes.POINTER(PlanInfo)]
_lib.tg_gate_workspace_bytes.restype = _sz
_lib.tg_gate_workspace_bytes.argtypes = [ctypes.POINTER(PlanInfo), _i32, _i32]
_lib.tg_gate_score.restype = _i32
_lib.tg_gate_score.argtypes = [_vp, _i64, _i32, _vp, _vp, _vp, _f32, _i32, _vp, ctypes.POINTER(PlanInfo), _f32, _vp,
                               _vp, _sz, _vp]
_lib.tg_gate_packed_w1_bytes.restype = _sz
_lib.tg_gate_packed_w1_bytes.argtypes = [_i32, _i32]
_lib.tg_gate_pack_w1.restype = _i32
_lib.tg_gate_pack_w1.argtypes = [_vp, _i32, _i32, _vp, _vp]
_lib.tg_gate_score_prepacked.restype = _i32
_lib.tg_gate_score_prepacked.argtypes = [_vp, _i64, _i32, _vp, _vp, _vp, _f32, _i32, _vp, ctypes.POINTER(PlanInfo), _f32,
                                         _vp, _vp, _sz, _vp]
_lib.tg_gate_score_prepacked_noalloc.restype = _i32
_lib.tg_gate_score_prepacked_noalloc.argtypes = [_vp, _i64, _i32, _vp, _vp, _vp, _f32, _i32, _vp,
                                                 ctypes.POINTER(PlanInfo), _f32, _vp, _vp]
_lib.tg_gate_noalloc_max_tiles.restype = _sz
_lib.tg_gate_noalloc_max_tiles.argtypes = []
_lib.tg_select_workspace_bytes.restype = _sz
_lib.tg_select_workspace_bytes.argtypes = [ctypes.POINTER(PlanInfo)]
_lib.tg_select_topk.restype = _i32
_lib.tg_select_topk.argtypes = [_vp, _vp, ctypes.POINTER(PlanInfo), _vp, _vp, _sz, _vp]
_lib.tg_compact_kept.restype = _i32
_lib.tg_compact_kept.argtypes = [_vp, _i64, _i64, _i32, ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.POINTER(_i64),
                                 ctypes.POINTER(_i64), ctypes.POINTER(_i64), _vp]
_lib.tg_gated_attention_prefill_gather.restype = _i32
_lib.tg_gated_attention_prefill_gather.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(PlanInfo), _i32,
                                                   _i32, _i32, _vp, _i64, _vp, _vp]
_lib.tg_gated_attention_prefill_gather_ws.restype = _i32
_lib.tg_gated_attention_prefill_gather_ws.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(PlanInfo),
                                                      _i32, _i32, _i32, _vp, _i64, _vp, _vp, _sz, _vp]
_lib.tg_gated_attention_prefill_query_tau_ws.restype = _i32
_lib.tg_gated_attention_prefill_query_tau_ws.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                         ctypes.POINTER(PlanInfo), _i32, _i32, _i32, _vp, _vp, _sz,
                                                         _vp]
_lib.tg_gated_attention_prefill_query_tau.restype = _i32
_lib.tg_gated_attention_prefill_query_tau.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(PlanInfo),
                                                      _i32, _i32, _i32, _vp, _vp]
_lib.tg_attention_workspace_status.restype = _i32
_lib.tg_attention_workspace_status.argtypes = [_vp, ctypes.POINTER(_i32), _vp]
_lib.tg_gated_attention_prefill_lse.restype = _i32
_lib.tg_gated_attention_prefill_lse.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(PlanInfo), _i32, _i32,
                                                _i32, _vp, _vp, _vp]
_lib.tg_attention_backward_workspace_bytes.restype = _sz
_lib.tg_attention_backward_workspace_bytes.argtypes = [ctypes.POINTER(PlanInfo), _i32, _i32, _i32]
_lib.tg_gated_attention_backward.restype = _i32
_lib.tg_gated_attention_backward.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(PlanInfo), _i32, _i32,
                                             _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.tg_decode_workspace_bytes.restype = _sz
_lib.tg_decode_workspace_bytes.argtypes = [_i32, _i32, _i32, _i64]
_lib.tg_gated_attention_decode.restype = _i32
_lib.tg_gated_attention_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i64, _i32, _i32, _i32, _vp,
                                           _vp, _sz, _vp]
_lib.tg_gated_attention_prefill.restype = _i32
_lib.tg_gated_attention_prefill.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(PlanInfo), _i32, _i32,
                                            _i32, _vp, _vp]
_lib.tg_attention_prefill_workspace_bytes.restype = _sz
_lib.tg_attention_prefill_workspace_bytes.argtypes = [ctypes.POINTER(PlanInfo), _i32, _i32, _i32]
_lib.tg_gated_attention_prefill_ws.restype = _i32
_lib.tg_gated_attention_prefill_ws.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(PlanInfo), _i32,
                                               _i32, _i32, _vp, _vp, _sz, _vp]


_lib.tg_gemm_bf16.restype = _i32
_lib.tg_gemm_bf16.argtypes = [_i32, _vp, _i64, _vp, _i64, _i64, _i32, _i32, _vp, _i64, _vp, _i64, _vp]
_lib.tg_rmsnorm_bf16.restype = _i32
_lib.tg_rmsnorm_bf16.argtypes = [_vp, _i64, _i64, _i32, _vp, _f32, _vp, _i64, _vp]
_lib.tg_rope_split_bf16.restype = _i32
_lib.tg_rope_split_bf16.argtypes = [_vp, _i64, _i64, _i32, _i32, _i32, _vp, _f32, _vp, _vp, _vp, _vp]
_lib.tg_decoder_layer_workspace_bytes.restype = _sz
_lib.tg_decoder_layer_workspace_bytes.argtypes = [_i64, _i32, _i32, _i32, _i32, _i32]
_lib.tg_decoder_layer.restype = _i32
_lib.tg_decoder_layer.argtypes = [_vp, _vp, _vp, _vp, ctypes.POINTER(PlanInfo), _i32, _i32, _i32, _i32, _i32, _f32,
                                  _f32, ctypes.POINTER(LayerWeights), _vp, _vp, _sz, _vp]


def library_path() -> str:
    return _LIB_PATH


def status_string(status: int) -> str:
    return _lib.tg_status_string(int(status)).decode()


def abi_version() -> int:
    return int(_lib.tg_abi_version())


def _check(status: int, where: str) -> None:
    if status != TG_OK:
        raise TokenGateError(int(status), where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(int(stream.cuda_stream))


def hip_runtimes_loaded() -> List[str]:
    """Distinct libamdhip64 files mapped into this process (there must be one)."""
    paths = set()
    with open("/proc/self/maps") as f:
        for ln in f:
            parts = ln.split()
            if len(parts) >= 6 and "libamdhip64" in parts[-1]:
                paths.add(os.path.realpath(parts[-1]))
    return sorted(paths)


# ----------------------------------------------------------------------------
# Segment plan
# ----------------------------------------------------------------------------


@dataclass
class Plan:
    info: PlanInfo
    table: np.ndarray  # host copy, int32 [n_seg, 8]
    table_dev: Optional[torch.Tensor]  # int32 [n_seg, 8] on the device

    @property
    def n_tokens(self) -> int:
        return int(self.info.n_tokens)

    @property
    def total_kept(self) -> int:
        return int(self.info.total_kept)

    @property
    def kept_offsets(self) -> np.ndarray:
        return np.concatenate([self.table[:, 5], [self.total_kept]]).astype(np.int64)


def plan_segments(seg_start: Sequence[int], doc_begin: Sequence[int], doc_end: Sequence[int],
                  k_budget: Sequence[int], device: Optional[torch.device] = None) -> Plan:
    """tg_plan_segments on host arrays; copies the table to ``device`` (None: host only)."""
    n_seg = len(doc_begin)
    ss = np.ascontiguousarray(seg_start, dtype=np.int32)
    db = np.ascontiguousarray(doc_begin, dtype=np.int32)
    de = np.ascontiguousarray(doc_end, dtype=np.int32)
    kb = np.ascontiguousarray(k_budget, dtype=np.int32)
    if ss.size != n_seg + 1 or de.size != n_seg or kb.size != n_seg:
        raise TokenGateError(-1, "plan_segments: array lengths")
    table = (Segment * max(n_seg, 1))()
    info = PlanInfo()
    st = _lib.tg_plan_segments(n_seg, ss.ctypes.data, db.ctypes.data, de.ctypes.data, kb.ctypes.data, table,
                               ctypes.byref(info))
    _check(st, "tg_plan_segments")
    host = np.frombuffer(bytearray(table), dtype=np.int32).reshape(-1, 8)[:n_seg].copy()
    dev = None
    if device is not None:
        dev = torch.from_numpy(host).to(device)
    return Plan(info=info, table=host, table_dev=dev)


def kept_count(n_doc: int, n_other: int, k: int) -> int:
    """tg_kept_count: min(k, n_doc) + n_other (-1 for a negative argument)."""
    return int(_lib.tg_kept_count(n_doc, n_other, k))


def plan_from(segments, device=None) -> Plan:
    """Plan of a workloads.Segments-like object (seg_start, doc_begin, doc_end, k_budget)."""
    return plan_segments(segments.seg_start, segments.doc_begin, segments.doc_end, segments.k_budget, device)


def _dev_table(plan: Plan) -> ctypes.c_void_p:
    if plan.table_dev is None:
        raise TokenGateError(-1, "plan has no device copy")
    return ctypes.c_void_p(plan.table_dev.data_ptr())


# ----------------------------------------------------------------------------
# Entry points
# ----------------------------------------------------------------------------


def gate_workspace_bytes(plan: Plan, d: int, h: int) -> int:
    return int(_lib.tg_gate_workspace_bytes(ctypes.byref(plan.info), d, h))


def select_workspace_bytes(plan: Plan) -> int:
    return int(_lib.tg_select_workspace_bytes(ctypes.byref(plan.info)))


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def gate_score(x: torch.Tensor, w1: torch.Tensor, b1: Optional[torch.Tensor], w2: torch.Tensor, b2: float, plan: Plan,
               rms_eps: float = 1e-6, scores: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """tg_gate_score.  x bf16 [n_tokens, >= d] (row stride = x.stride(0)), w1 bf16 [h, d]."""
    h, d = w1.shape
    if scores is None:
        scores = torch.empty(plan.n_tokens, dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = _workspace(gate_workspace_bytes(plan, d, h), x.device)
    st = _lib.tg_gate_score(_ptr(x), x.stride(0), d, _ptr(w1), _ptr(b1), _ptr(w2), float(b2), h, _dev_table(plan),
                            ctypes.byref(plan.info), float(rms_eps), _ptr(scores), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "tg_gate_score")
    return scores


def gate_pack_w1(w1: torch.Tensor, stream=None) -> torch.Tensor:
    """tg_gate_pack_w1: W1 bf16 [h, d] -> its fragment-ordered copy (opaque, for gate_score_prepacked)."""
    h, d = w1.shape
    out = torch.empty(int(_lib.tg_gate_packed_w1_bytes(d, h)), dtype=torch.uint8, device=w1.device)
    _check(_lib.tg_gate_pack_w1(_ptr(w1), d, h, _ptr(out), _stream(stream)), "tg_gate_pack_w1")
    return out


def gate_score_prepacked(x: torch.Tensor, w1_packed: torch.Tensor, h: int, b1: Optional[torch.Tensor],
                         w2: torch.Tensor, b2: float, plan: Plan, rms_eps: float = 1e-6,
                         scores: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                         stream=None) -> torch.Tensor:
    """tg_gate_score_prepacked: gate_score with W1 packed by gate_pack_w1."""
    d = int(w1_packed.numel() * w1_packed.element_size()) // (2 * h)
    if scores is None:
        scores = torch.empty(plan.n_tokens, dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = _workspace(gate_workspace_bytes(plan, d, h), x.device)
    st = _lib.tg_gate_score_prepacked(_ptr(x), x.stride(0), d, _ptr(w1_packed), _ptr(b1), _ptr(w2), float(b2), h,
                                      _dev_table(plan), ctypes.byref(plan.info), float(rms_eps), _ptr(scores),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "tg_gate_score_prepacked")
    return scores


def gate_noalloc_max_tiles() -> int:
    """tg_gate_noalloc_max_tiles: prompts x 64-row document tiles the no-allocation gate supports."""
    return int(_lib.tg_gate_noalloc_max_tiles())


def gate_score_prepacked_noalloc(x: torch.Tensor, w1_packed: torch.Tensor, h: int, b1: Optional[torch.Tensor],
                                 w2: torch.Tensor, b2: float, plan: Plan, scores: torch.Tensor,
                                 rms_eps: float = 1e-6, stream=None) -> torch.Tensor:
    """tg_gate_score_prepacked_noalloc: gate_score_prepacked without a workspace (the library's fixed scratch);
    the caller passes the output, so nothing is allocated."""
    d = int(w1_packed.numel() * w1_packed.element_size()) // (2 * h)
    st = _lib.tg_gate_score_prepacked_noalloc(_ptr(x), x.stride(0), d, _ptr(w1_packed), _ptr(b1), _ptr(w2),
                                              float(b2), h, _dev_table(plan), ctypes.byref(plan.info),
                                              float(rms_eps), _ptr(scores), _stream(stream))
    _check(st, "tg_gate_score_prepacked_noalloc")
    return scores


def select_topk(scores: torch.Tensor, plan: Plan, kept_idx: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """tg_select_topk -> int32 [total_kept] ascending global token indices."""
    if kept_idx is None:
        kept_idx = torch.empty(max(plan.total_kept, 1), dtype=torch.int32, device=scores.device)[:plan.total_kept]
    if workspace is None:
        workspace = _workspace(select_workspace_bytes(plan), scores.device)
    st = _lib.tg_select_topk(_ptr(scores), _dev_table(plan), ctypes.byref(plan.info), _ptr(kept_idx),
                             _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "tg_select_topk")
    return kept_idx


def compact_kept(kept_idx: torch.Tensor, pairs: Sequence[Tuple[torch.Tensor, torch.Tensor]], stream=None) -> None:
    """tg_compact_kept: for every (src, dst), dst[r] = src[kept_idx[r]] (rows = dim 0)."""
    n = len(pairs)
    srcs = (_vp * n)(*[p[0].data_ptr() for p in pairs])
    dsts = (_vp * n)(*[p[1].data_ptr() for p in pairs])
    rb = (_i64 * n)(*[math.prod(p[0].shape[1:]) * p[0].element_size() for p in pairs])  # bytes of one row
    ss = (_i64 * n)(*[p[0].stride(0) * p[0].element_size() for p in pairs])
    ds = (_i64 * n)(*[p[1].stride(0) * p[1].element_size() for p in pairs])
    n_src = min(p[0].shape[0] for p in pairs)
    st = _lib.tg_compact_kept(_ptr(kept_idx), kept_idx.numel(), n_src, n, srcs, dsts, rb, ss, ds, _stream(stream))
    _check(st, "tg_compact_kept")


def attention_prefill_workspace_bytes(plan: Plan, hq: int, hkv: int, head_dim: int) -> int:
    """tg_attention_prefill_workspace_bytes: 0 when no query tile is split."""
    return int(_lib.tg_attention_prefill_workspace_bytes(ctypes.byref(plan.info), hq, hkv, head_dim))


def attention_prefill_workspace(plan: Plan, hq: int, hkv: int, head_dim: int, device) -> torch.Tensor:
    """A zero-filled workspace for gated_attention_prefill(..., workspace=)."""
    return torch.zeros(max(attention_prefill_workspace_bytes(plan, hq, hkv, head_dim), 256), dtype=torch.uint8,
                       device=device)


def attention_workspace_status(workspace: torch.Tensor, stream=None) -> int:
    """tg_attention_workspace_status: 0 while every call on the split-tile workspace merged normally; bit 1 if a
    call found its counters already set, bit 2 if a wait ran out (those calls wrote NaN rows).  Synchronises the
    stream."""
    word = _i32(0)
    _check(_lib.tg_attention_workspace_status(_ptr(workspace), ctypes.byref(word), _stream(stream)),
           "tg_attention_workspace_status")
    return int(word.value)


def gated_attention_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, key_score: Optional[torch.Tensor],
                            tau: Optional[torch.Tensor], gain: Optional[torch.Tensor], plan: Plan,
                            out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                            stream=None) -> torch.Tensor:
    """tg_gated_attention_prefill.  q [M, hq, D], k/v [M, hkv, D] bf16 contiguous.  With a workspace (from
    attention_prefill_workspace) it calls tg_gated_attention_prefill_ws, which may split long query tiles."""
    m, hq, dh = q.shape
    hkv = k.shape[1]
    if out is None:
        out = torch.empty_like(q)
    if workspace is not None:
        st = _lib.tg_gated_attention_prefill_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(key_score), _ptr(tau), _ptr(gain),
                                                _dev_table(plan), ctypes.byref(plan.info), hq, hkv, dh, _ptr(out),
                                                _ptr(workspace), workspace.numel() * workspace.element_size(),
                                                _stream(stream))
        _check(st, "tg_gated_attention_prefill_ws")
        return out
    st = _lib.tg_gated_attention_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(key_score), _ptr(tau), _ptr(gain),
                                         _dev_table(plan), ctypes.byref(plan.info), hq, hkv, dh, _ptr(out),
                                         _stream(stream))
    _check(st, "tg_gated_attention_prefill")
    return out


def gated_attention_prefill_gather(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                   key_score: Optional[torch.Tensor], tau: Optional[torch.Tensor],
                                   gain: Optional[torch.Tensor], plan: Plan, kept_idx: torch.Tensor,
                                   out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                                   stream=None) -> torch.Tensor:
    """tg_gated_attention_prefill_gather.  q [N, hq, D], k/v [N, hkv, D] bf16
    contiguous over every token; kept_idx int32 [M]; returns out [M, hq, D].  With a
    workspace (attention_prefill_workspace) it calls tg_gated_attention_prefill_gather_ws."""
    n_src, hq, dh = q.shape
    hkv = k.shape[1]
    if out is None:
        out = torch.empty((plan.total_kept, hq, dh), dtype=q.dtype, device=q.device)
    if workspace is not None:
        st = _lib.tg_gated_attention_prefill_gather_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(key_score), _ptr(tau),
                                                       _ptr(gain), _dev_table(plan), ctypes.byref(plan.info), hq,
                                                       hkv, dh, _ptr(kept_idx), n_src, _ptr(out), _ptr(workspace),
                                                       workspace.numel() * workspace.element_size(), _stream(stream))
        _check(st, "tg_gated_attention_prefill_gather_ws")
        return out
    st = _lib.tg_gated_attention_prefill_gather(_ptr(q), _ptr(k), _ptr(v), _ptr(key_score), _ptr(tau), _ptr(gain),
                                                _dev_table(plan), ctypes.byref(plan.info), hq, hkv, dh,
                                                _ptr(kept_idx), n_src, _ptr(out), _stream(stream))
    _check(st, "tg_gated_attention_prefill_gather")
    return out


def gated_attention_prefill_query_tau(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                      key_score: Optional[torch.Tensor], sigma: torch.Tensor,
                                      gain: Optional[torch.Tensor], positions: torch.Tensor, plan: Plan,
                                      out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                                      stream=None) -> torch.Tensor:
    """tg_gated_attention_prefill_query_tau.  As gated_attention_prefill, with
    sigma fp32 [hq] and positions int32 [M] (original positions of the kept rows).  With a
    workspace (attention_prefill_workspace) it calls tg_gated_attention_prefill_query_tau_ws."""
    m, hq, dh = q.shape
    hkv = k.shape[1]
    if out is None:
        out = torch.empty_like(q)
    if workspace is not None:
        st = _lib.tg_gated_attention_prefill_query_tau_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(key_score), _ptr(sigma),
                                                          _ptr(gain), _ptr(positions), _dev_table(plan),
                                                          ctypes.byref(plan.info), hq, hkv, dh, _ptr(out),
                                                          _ptr(workspace),
                                                          workspace.numel() * workspace.element_size(),
                                                          _stream(stream))
        _check(st, "tg_gated_attention_prefill_query_tau_ws")
        return out
    st = _lib.tg_gated_attention_prefill_query_tau(_ptr(q), _ptr(k), _ptr(v), _ptr(key_score), _ptr(sigma),
                                                   _ptr(gain), _ptr(positions), _dev_table(plan),
                                                   ctypes.byref(plan.info), hq, hkv, dh, _ptr(out), _stream(stream))
    _check(st, "tg_gated_attention_prefill_query_tau")
    return out


def gated_attention_prefill_lse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                key_score: Optional[torch.Tensor], tau: Optional[torch.Tensor],
                                gain: Optional[torch.Tensor], plan: Plan, out: Optional[torch.Tensor] = None,
                                lse: Optional[torch.Tensor] = None, stream=None):
    """tg_gated_attention_prefill_lse: returns (out [M, hq, D] bf16, lse [M, hq] fp32)."""
    m, hq, dh = q.shape
    hkv = k.shape[1]
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((m, hq), dtype=torch.float32, device=q.device)
    st = _lib.tg_gated_attention_prefill_lse(_ptr(q), _ptr(k), _ptr(v), _ptr(key_score), _ptr(tau), _ptr(gain),
                                             _dev_table(plan), ctypes.byref(plan.info), hq, hkv, dh, _ptr(out),
                                             _ptr(lse), _stream(stream))
    _check(st, "tg_gated_attention_prefill_lse")
    return out, lse


def attention_backward_workspace_bytes(plan: Plan, hq: int, hkv: int, head_dim: int) -> int:
    return int(_lib.tg_attention_backward_workspace_bytes(ctypes.byref(plan.info), hq, hkv, head_dim))


def gated_attention_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, key_score: Optional[torch.Tensor],
                             tau: Optional[torch.Tensor], gain: Optional[torch.Tensor], plan: Plan,
                             out: torch.Tensor, dout: torch.Tensor, lse: torch.Tensor,
                             workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """tg_gated_attention_backward: returns fp32 dq, dk, dv, ds, dgain, dtau."""
    m, hq, dh = q.shape
    hkv = k.shape[1]
    dev = q.device
    g = {"dq": torch.empty((m, hq, dh), dtype=torch.float32, device=dev),
         "dk": torch.empty((m, hkv, dh), dtype=torch.float32, device=dev),
         "dv": torch.empty((m, hkv, dh), dtype=torch.float32, device=dev),
         "ds": torch.empty(m, dtype=torch.float32, device=dev),
         "dgain": torch.empty(hq, dtype=torch.float32, device=dev),
         "dtau": torch.empty(hq, dtype=torch.float32, device=dev)}
    if workspace is None:
        workspace = _workspace(attention_backward_workspace_bytes(plan, hq, hkv, dh), dev)
    st = _lib.tg_gated_attention_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(key_score), _ptr(tau), _ptr(gain),
                                          _dev_table(plan), ctypes.byref(plan.info), hq, hkv, dh, _ptr(out),
                                          _ptr(dout), _ptr(lse), _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]),
                                          _ptr(g["ds"]), _ptr(g["dgain"]), _ptr(g["dtau"]), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "tg_gated_attention_backward")
    return g


def decode_workspace_bytes(batch: int, hq: int, head_dim: int, cache_rows: int) -> int:
    return int(_lib.tg_decode_workspace_bytes(batch, hq, head_dim, cache_rows))


def gated_attention_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           key_score: Optional[torch.Tensor], tau: Optional[torch.Tensor],
                           gain: Optional[torch.Tensor], lens: torch.Tensor, out: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """tg_gated_attention_decode.  q [B, hq, D]; k_cache / v_cache [B, cap, hkv, D]
    bf16 contiguous; key_score [B, cap] fp32; tau [hq] or [B, hq] (per query);
    lens int32 [B]; returns out [B, hq, D]."""
    bsz, hq, dh = q.shape
    cap, hkv = k_cache.shape[1], k_cache.shape[2]
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = _workspace(decode_workspace_bytes(bsz, hq, dh, cap), q.device)
    per_query = 1 if tau is not None and tau.dim() == 2 else 0
    st = _lib.tg_gated_attention_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(key_score), _ptr(tau), per_query,
                                        _ptr(gain), _ptr(lens), bsz, cap, hq, hkv, dh, _ptr(out), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "tg_gated_attention_decode")
    return out


# ----------------------------------------------------------------------------
# Dense decoder-layer support
# ----------------------------------------------------------------------------


def gemm_bf16(x: torch.Tensor, w: torch.Tensor, epilogue: int = GEMM_STORE, residual: Optional[torch.Tensor] = None,
              out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """tg_gemm_bf16: out = x . w^T (+ residual | SwiGLU).  x [m, k], w [n, k] bf16 (row strides honoured)."""
    m, k = x.shape
    n = w.shape[0]
    n_out = n // 2 if epilogue == GEMM_SWIGLU else n
    if out is None:
        out = torch.empty((m, n_out), dtype=torch.bfloat16, device=x.device)
    st = _lib.tg_gemm_bf16(epilogue, _ptr(x), x.stride(0), _ptr(w), w.stride(0), m, n, k, _ptr(residual),
                           residual.stride(0) if residual is not None else 0, _ptr(out), out.stride(0),
                           _stream(stream))
    _check(st, "tg_gemm_bf16")
    return out


def rmsnorm_bf16(x: torch.Tensor, weight: torch.Tensor, eps: float = 1e-6, out: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    m, d = x.shape
    if out is None:
        out = torch.empty_like(x)
    st = _lib.tg_rmsnorm_bf16(_ptr(x), x.stride(0), m, d, _ptr(weight), float(eps), _ptr(out), out.stride(0),
                              _stream(stream))
    _check(st, "tg_rmsnorm_bf16")
    return out


def rope_split_bf16(qkv: torch.Tensor, hq: int, hkv: int, head_dim: int, positions: torch.Tensor,
                    theta: float = 1e6, stream=None):
    m = qkv.shape[0]
    q = torch.empty((m, hq, head_dim), dtype=torch.bfloat16, device=qkv.device)
    k = torch.empty((m, hkv, head_dim), dtype=torch.bfloat16, device=qkv.device)
    v = torch.empty_like(k)
    st = _lib.tg_rope_split_bf16(_ptr(qkv), qkv.stride(0), m, hq, hkv, head_dim, _ptr(positions), float(theta),
                                 _ptr(q), _ptr(k), _ptr(v), _stream(stream))
    _check(st, "tg_rope_split_bf16")
    return q, k, v


def decoder_layer_workspace_bytes(m: int, d: int, hq: int, hkv: int, head_dim: int, f: int) -> int:
    return int(_lib.tg_decoder_layer_workspace_bytes(m, d, hq, hkv, head_dim, f))


def decoder_layer(hidden: torch.Tensor, positions: torch.Tensor, key_score: Optional[torch.Tensor], plan: Plan,
                  weights: LayerWeights, d: int, hq: int, hkv: int, head_dim: int, f: int,
                  workspace: torch.Tensor, rms_eps: float = 1e-6, rope_theta: float = 1e6,
                  post_attn_norm: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """tg_decoder_layer: hidden [total_kept, d] bf16 updated in place."""
    st = _lib.tg_decoder_layer(_ptr(hidden), _ptr(positions), _ptr(key_score), _dev_table(plan),
                               ctypes.byref(plan.info), d, hq, hkv, head_dim, f, float(rms_eps), float(rope_theta),
                               ctypes.byref(weights), _ptr(post_attn_norm), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "tg_decoder_layer")
    return hidden
