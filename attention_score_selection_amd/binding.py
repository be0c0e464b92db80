"""ctypes binding of ``libtsel.so`` (declared in ``include/tsel.h``).

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream.  If the library is
not built, every call raises; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# TSEL_LIBRARY names another build of the same library (the host-sanitizer
# build the CPU tests use); by default the in-tree libtsel.so.
LIB_PATH = os.environ.get("TSEL_LIBRARY") or os.path.join(_HERE, "libtsel.so")

TSEL_OK, TSEL_EINVAL, TSEL_EUNSUPPORTED, TSEL_EWORKSPACE, TSEL_EHIP = 0, -1, -2, -3, -4
TSEL_F32, TSEL_F16, TSEL_BF16, TSEL_FP8_E4M3 = 0, 1, 2, 3
MASKS = {"full": 0, "causal": 1, "blockdiag": 2}
TSEL_OP_LSE, TSEL_OP_COLSCORE, TSEL_OP_TOPK, TSEL_OP_COMPACT, TSEL_OP_MROPE = 0, 1, 2, 3, 4
EXPORTS = ("tsel_lse", "tsel_colscore", "tsel_colscore_noalloc", "tsel_budget_topk", "tsel_compact", "tsel_mrope_positions",
           "tsel_attention_fwd", "tsel_budget_mass",
           "tsel_workspace_size", "tsel_last_error", "tsel_version")

_DTYPES = {torch.float32: TSEL_F32, torch.float16: TSEL_F16, torch.bfloat16: TSEL_BF16,
           torch.float8_e4m3fn: TSEL_FP8_E4M3}
_P = ctypes.c_void_p
_I32P = ctypes.POINTER(ctypes.c_int32)


class TselError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"tsel error {code}: {message}")
        self.code = code


class CLayout(ctypes.Structure):
    _fields_ = [("num_reqs", ctypes.c_int32), ("num_images", ctypes.c_int32),
                ("total_tokens", ctypes.c_int32), ("max_seqlen", ctypes.c_int32),
                ("cu_seqlens", _P), ("cu_images", _P), ("img_start", _P), ("img_hw", _P),
                ("cu_cands", _P),
                ("cu_seqlens_h", _P), ("cu_images_h", _P), ("img_start_h", _P), ("img_hw_h", _P),
                ("cu_cands_h", _P)]


class CAttn(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("num_heads_q", ctypes.c_int32),
                ("num_heads_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("q", _P), ("q_stride_tok", ctypes.c_int64), ("q_stride_head", ctypes.c_int64),
                ("k", _P), ("k_stride_tok", ctypes.c_int64), ("k_stride_head", ctypes.c_int64),
                ("mask", ctypes.c_int), ("softmax_scale", ctypes.c_float)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the library once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.tsel_version.restype = ctypes.c_int
        L.tsel_last_error.restype = ctypes.c_char_p
        L.tsel_workspace_size.restype = ctypes.c_size_t
        L.tsel_workspace_size.argtypes = [ctypes.c_int, ctypes.POINTER(CAttn), ctypes.POINTER(CLayout)]
        L.tsel_lse.restype = ctypes.c_int
        L.tsel_lse.argtypes = [ctypes.POINTER(CAttn), ctypes.POINTER(CLayout), _P, _P, ctypes.c_size_t, _P]
        L.tsel_colscore.restype = ctypes.c_int
        L.tsel_colscore.argtypes = [ctypes.POINTER(CAttn), ctypes.POINTER(CLayout), _P, _P, _P,
                                    ctypes.c_size_t, _P]
        L.tsel_colscore_noalloc.restype = ctypes.c_int
        L.tsel_colscore_noalloc.argtypes = [ctypes.POINTER(CAttn), ctypes.POINTER(CLayout), _P, _P, _P]
        L.tsel_budget_topk.restype = ctypes.c_int
        L.tsel_budget_topk.argtypes = [ctypes.POINTER(CLayout), _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.tsel_budget_mass.restype = ctypes.c_int
        L.tsel_budget_mass.argtypes = [ctypes.POINTER(CLayout), _P, _P, _P, _P, _P, _P, _P]
        L.tsel_compact.restype = ctypes.c_int
        L.tsel_compact.argtypes = [ctypes.POINTER(CLayout), _P, _P, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int32, _P, ctypes.c_int64, _P, _P, _P, _P, _P,
                                   ctypes.c_size_t, _P]
        L.tsel_attention_fwd.restype = ctypes.c_int
        L.tsel_attention_fwd.argtypes = [ctypes.POINTER(CAttn), ctypes.POINTER(CLayout), _P,
                                         ctypes.c_int64, ctypes.c_int64, _P, ctypes.c_int64,
                                         ctypes.c_int64, _P, _P]
        L.tsel_mrope_positions.restype = ctypes.c_int
        L.tsel_mrope_positions.argtypes = [ctypes.POINTER(CLayout), _P, _P, ctypes.c_int32, _P, _P,
                                           ctypes.c_size_t, _P]
        _lib = L
    return _lib


def _check(rc: int):
    if rc != TSEL_OK:
        raise TselError(rc, lib().tsel_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


class Layout:
    """Token layout with the host mirrors and device copies the C-ABI wants.

    Arrays follow ``tsel_layout_t``: cu_seqlens [B+1], cu_images [B+1],
    img_start [S], img_hw [S, 2], cu_cands [S+1].
    """

    def __init__(self, cu_seqlens, cu_images, img_start, img_hw, cu_cands, device="cuda"):
        self.h = {name: np.ascontiguousarray(np.asarray(a, np.int32).reshape(-1))
                  for name, a in (("cu_seqlens", cu_seqlens), ("cu_images", cu_images),
                                  ("img_start", img_start), ("img_hw", img_hw),
                                  ("cu_cands", cu_cands))}
        self.device = torch.device(device)
        if self.device.type == "cuda":
            self.d = {k: torch.from_numpy(v.copy()).to(self.device) for k, v in self.h.items()}
        else:
            self.d = None
        self.B = len(self.h["cu_seqlens"]) - 1
        self.S = len(self.h["img_start"])
        self.T = int(self.h["cu_seqlens"][-1])
        self.N = int(self.h["cu_cands"][-1])
        c = CLayout()
        c.num_reqs, c.num_images, c.total_tokens = self.B, self.S, self.T
        c.max_seqlen = int(np.diff(self.h["cu_seqlens"]).max(initial=0))
        for name in self.h:
            setattr(c, name + "_h", self.h[name].ctypes.data if self.h[name].size else None)
            setattr(c, name, self.d[name].data_ptr() if (self.d and self.h[name].size) else None)
        self.c = c

    @classmethod
    def from_problem(cls, prob, device="cuda") -> "Layout":
        return cls(prob.cu_seqlens, prob.cu_images, prob.img_start, prob.img_hw, prob.cu_cands,
                   device)

    def pool_sizes(self):
        ci, cc = self.h["cu_images"], self.h["cu_cands"]
        return [int(cc[ci[b + 1]] - cc[ci[b]]) for b in range(self.B)]


def make_attn(q: torch.Tensor, k: torch.Tensor, mask: str, softmax_scale: float = 0.0) -> CAttn:
    if q.dim() != 3 or k.dim() != 3 or q.stride(2) != 1 or k.stride(2) != 1:
        raise ValueError("q and k must be [T, H, d] with a contiguous last dimension")
    if q.dtype != k.dtype or q.dtype not in _DTYPES:
        raise ValueError("q and k must share one dtype among float32, float16, bfloat16, "
                         "float8_e4m3fn")
    a = CAttn()
    a.dtype = _DTYPES[q.dtype]
    a.num_heads_q, a.num_heads_kv, a.head_dim = q.shape[1], k.shape[1], q.shape[2]
    a.q, a.q_stride_tok, a.q_stride_head = q.data_ptr(), q.stride(0), q.stride(1)
    a.k, a.k_stride_tok, a.k_stride_head = k.data_ptr(), k.stride(0), k.stride(1)
    a.mask = MASKS[mask]
    a.softmax_scale = float(softmax_scale)
    return a


def tsel_workspace_size(op: int, layout: Layout, q=None, k=None, mask="causal",
                        softmax_scale: float = 0.0) -> int:
    attn = make_attn(q, k, mask, softmax_scale) if q is not None else None
    n = lib().tsel_workspace_size(op, ctypes.byref(attn) if attn is not None else None,
                                  ctypes.byref(layout.c))
    if n == ctypes.c_size_t(-1).value:
        raise TselError(TSEL_EINVAL, lib().tsel_last_error().decode())
    return int(n)


def _workspace(need: int, workspace: Optional[torch.Tensor], device) -> torch.Tensor:
    """The caller's workspace if it is large enough, else a new one."""
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=device)
    return workspace


def tsel_lse(q: torch.Tensor, k: torch.Tensor, layout: Layout, mask: str,
             softmax_scale: float = 0.0, out: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-row softmax LSE, fp32 [Hq, T]."""
    attn = make_attn(q, k, mask, softmax_scale)
    if out is None:
        out = torch.empty((q.shape[1], layout.T), dtype=torch.float32, device=q.device)
    need = tsel_workspace_size(TSEL_OP_LSE, layout, q, k, mask, softmax_scale)
    ws = _workspace(need, workspace, q.device) if need > 0 else None
    _check(lib().tsel_lse(ctypes.byref(attn), ctypes.byref(layout.c), _ptr(out), _ptr(ws),
                          0 if ws is None else ws.numel() * ws.element_size(), _stream(q.device)))
    return out


def tsel_colscore(q: torch.Tensor, k: torch.Tensor, layout: Layout, mask: str, lse: torch.Tensor,
                  softmax_scale: float = 0.0, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Importance score per candidate, fp32 [N]."""
    attn = make_attn(q, k, mask, softmax_scale)
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [Hq, T] tensor")
    if out is None:
        out = torch.empty((layout.N,), dtype=torch.float32, device=q.device)
    need = tsel_workspace_size(TSEL_OP_COLSCORE, layout, q, k, mask, softmax_scale)
    workspace = _workspace(need, workspace, q.device)
    _check(lib().tsel_colscore(ctypes.byref(attn), ctypes.byref(layout.c), _ptr(lse), _ptr(out),
                               _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _stream(q.device)))
    return out


def tsel_colscore_noalloc(q: torch.Tensor, k: torch.Tensor, layout: Layout, mask: str, lse: torch.Tensor,
                          softmax_scale: float = 0.0, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """tsel_colscore with the library's static device scratch (no workspace)."""
    attn = make_attn(q, k, mask, softmax_scale)
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [Hq, T] tensor")
    if out is None:
        out = torch.empty((layout.N,), dtype=torch.float32, device=q.device)
    _check(lib().tsel_colscore_noalloc(ctypes.byref(attn), ctypes.byref(layout.c), _ptr(lse), _ptr(out),
                                       _stream(q.device)))
    return out


def tsel_budget_topk(layout: Layout, score: torch.Tensor, keep_ratio: Sequence[float],
                     out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Keep flags (uint8 [N]) and k per pool (numpy int32 [B])."""
    ratios = np.ascontiguousarray(np.asarray(keep_ratio, np.float64).reshape(-1))
    if ratios.size != layout.B:
        raise ValueError("one keep ratio per request is required")
    k_h = np.zeros(layout.B, np.int32)
    if out is None:
        out = torch.empty((layout.N,), dtype=torch.uint8, device=score.device)
    need = tsel_workspace_size(TSEL_OP_TOPK, layout)
    ws = _workspace(need, workspace, score.device) if need > 0 else None
    _check(lib().tsel_budget_topk(ctypes.byref(layout.c), _ptr(score), ratios.ctypes.data,
                                  k_h.ctypes.data, _ptr(out), _ptr(ws),
                                  0 if ws is None else ws.numel() * ws.element_size(), _stream(score.device)))
    return out, k_h


def tsel_budget_mass(layout: Layout, score: torch.Tensor, tau: Sequence[float], r_min: Sequence[float],
                     r_max: Sequence[float], out: Optional[torch.Tensor] = None,
                     k_out: Optional[torch.Tensor] = None):
    """Input-dependent budget: keep flags (uint8 [N]) and k per pool (device
    int32 [B]; ``.cpu()`` it to size the compaction)."""
    arrs = [np.ascontiguousarray(np.asarray(x, np.float64).reshape(-1)) for x in (tau, r_min, r_max)]
    if any(a.size != layout.B for a in arrs):
        raise ValueError("one tau, r_min and r_max per request are required")
    if out is None:
        out = torch.empty((layout.N,), dtype=torch.uint8, device=score.device)
    if k_out is None:
        k_out = torch.empty((max(layout.B, 1),), dtype=torch.int32, device=score.device)
    _check(lib().tsel_budget_mass(ctypes.byref(layout.c), _ptr(score), arrs[0].ctypes.data, arrs[1].ctypes.data,
                                  arrs[2].ctypes.data, _ptr(k_out), _ptr(out), _stream(score.device)))
    return out, k_out[:layout.B]


def tsel_compact(layout: Layout, keep: torch.Tensor, k_per_pool, emb: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, outputs: Optional[dict] = None) -> dict:
    """Stable compaction: token_idx [T_out], spatial [T_out, 3], cu_seqlens [B+1],
    img_counts [S] and (if emb is given) emb [T_out, D]."""
    dev = keep.device
    t_out = layout.T - layout.N + int(np.sum(k_per_pool))
    o = outputs if outputs is not None else {}
    if "token_idx" not in o:
        o["token_idx"] = torch.empty((t_out,), dtype=torch.int32, device=dev)
        o["spatial"] = torch.empty((t_out, 3), dtype=torch.int32, device=dev)
        o["cu_seqlens"] = torch.empty((layout.B + 1,), dtype=torch.int32, device=dev)
        o["img_counts"] = torch.empty((max(layout.S, 1),), dtype=torch.int32, device=dev)
    emb_ptr = out_ptr = None
    emb_stride = row_bytes = out_stride = 0
    if emb is not None:
        if emb.dim() != 2 or emb.stride(1) != 1:
            raise ValueError("emb must be [T, D] with a contiguous last dimension")
        if "emb" not in o:
            o["emb"] = torch.empty((t_out, emb.shape[1]), dtype=emb.dtype, device=dev)
        es = emb.element_size()
        emb_ptr, emb_stride, row_bytes = emb.data_ptr(), emb.stride(0) * es, emb.shape[1] * es
        out_ptr, out_stride = o["emb"].data_ptr(), o["emb"].stride(0) * es
    need = tsel_workspace_size(TSEL_OP_COMPACT, layout)
    workspace = _workspace(need, workspace, dev)
    _check(lib().tsel_compact(ctypes.byref(layout.c), _ptr(keep), emb_ptr, emb_stride, row_bytes,
                              t_out, out_ptr, out_stride, _ptr(o["token_idx"]), _ptr(o["spatial"]),
                              _ptr(o["cu_seqlens"]), _ptr(o["img_counts"]), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(dev)))
    return o


def tsel_attention_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, layout: Layout, mask: str,
                       softmax_scale: float = 0.0, out: Optional[torch.Tensor] = None,
                       lse: Optional[torch.Tensor] = None):
    """Attention forward: out [T, Hq, d] in q's dtype and the LSE fp32 [Hq, T]."""
    attn = make_attn(q, k, mask, softmax_scale)
    if v.dim() != 3 or v.dtype != q.dtype or v.stride(2) != 1 or v.shape != k.shape:
        raise ValueError("v must be [T, Hkv, d] like k, with a contiguous last dimension")
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((q.shape[1], layout.T), dtype=torch.float32, device=q.device)
    _check(lib().tsel_attention_fwd(ctypes.byref(attn), ctypes.byref(layout.c), _ptr(v), v.stride(0),
                                    v.stride(1), _ptr(out), out.stride(0), out.stride(1), _ptr(lse),
                                    _stream(q.device)))
    return out, lse


def tsel_mrope_positions(layout: Layout, compact: dict, out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Rotary (t, h, w) positions [T_out, 3] of the compacted sequence, from
    tsel_compact's token_idx and spatial outputs."""
    tok, sp = compact["token_idx"], compact["spatial"]
    dev = tok.device
    n = int(tok.numel())
    if out is None:
        out = torch.empty((n, 3), dtype=torch.int32, device=dev)
    need = tsel_workspace_size(TSEL_OP_MROPE, layout)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty((max(need, 4),), dtype=torch.uint8, device=dev)
    _check(lib().tsel_mrope_positions(ctypes.byref(layout.c), _ptr(tok), _ptr(sp), n, _ptr(out),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(dev)))
    return out


def select(q: torch.Tensor, k: torch.Tensor, layout: Layout, mask: str, keep_ratio,
           emb: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
           softmax_scale: float = 0.0, mass=None) -> dict:
    """The whole path: LSE (unless supplied) -> scores -> budget -> compaction
    -> rotary positions of the compacted sequence.  The budget is the fixed
    ratio top-k (keep_ratio), or with ``mass=(tau, r_min, r_max)`` (per-pool
    sequences) the input-dependent one; its k per pool is then copied to the
    host to size the compaction (one synchronisation)."""
    if lse is None:
        lse = tsel_lse(q, k, layout, mask, softmax_scale)
    score = tsel_colscore(q, k, layout, mask, lse, softmax_scale)
    if mass is None:
        keep, ks = tsel_budget_topk(layout, score, keep_ratio)
    else:
        keep, kd = tsel_budget_mass(layout, score, *mass)
        ks = kd.cpu().numpy()
    comp = tsel_compact(layout, keep, ks, emb)
    comp["positions"] = tsel_mrope_positions(layout, comp)
    return dict(lse=lse, score=score, keep=keep, k=ks, compact=comp)
