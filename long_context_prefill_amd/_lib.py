"""Thin ctypes binding of libs2o.so (declared in include/s2o.h).

Argument marshalling only: every step of the path runs in the HIP library.
PyTorch supplies device memory (tensors, workspaces) and the current stream.
There is no fallback: if the library is missing or a call fails, an exception
is raised.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libs2o.so")

# every symbol include/s2o.h declares
EXPORTS = ("s2o_check_problem", "s2o_list_entries", "s2o_list_offset",
           "s2o_score_workspace_bytes", "s2o_score", "s2o_score_noalloc", "s2o_build_index_workspace_bytes",
           "s2o_build_index", "s2o_attn_fwd", "dense_attn_fwd", "s2o_status_string")

STATUS = {0: "S2O_OK", -1: "S2O_ERR_INVALID_ARG", -2: "S2O_ERR_UNSUPPORTED",
          -3: "S2O_ERR_WORKSPACE", -4: "S2O_ERR_HIP"}
F32, BF16 = 0, 1


class S2OError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({msg})")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32),
                ("heads_kv", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("seg_len", ctypes.c_int32),
                ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("scale", ctypes.c_float), ("list_granularity", ctypes.c_int32)]

    def astuple(self):
        return tuple(getattr(self, f) for f, _ in self._fields_)


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(hipcc, gfx950); there is no CPU fallback")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(Problem)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        sig = {
            "s2o_check_problem": (ctypes.c_int, [P]),
            "s2o_list_entries": (i64, [P]),
            "s2o_list_offset": (i64, [P, i32, i32, i32]),
            "s2o_score_workspace_bytes": (sz, [P]),
            "s2o_score": (ctypes.c_int, [P, vp, vp, vp, vp, sz, vp]),
            "s2o_score_noalloc": (ctypes.c_int, [P, vp, vp, vp, vp]),
            "s2o_build_index_workspace_bytes": (sz, [P]),
            "s2o_build_index": (ctypes.c_int, [P, vp, vp, vp, sz, vp]),
            "s2o_attn_fwd": (ctypes.c_int, [P, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp]),
            "dense_attn_fwd": (ctypes.c_int, [P, vp, vp, vp, vp, vp]),
            "s2o_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _raise(fn: str, st: int):
    if st != 0:
        raise S2OError(fn, st, lib().s2o_status_string(st).decode())


LISTS = {"tile": 0, "segment": 1, "tile_blocks": 2, "segment_blocks": 3}
QUERY_PERMUTATION = 4
SHARE_GQA = 8
LISTS_PER_TILE, LISTS_PER_SEGMENT = LISTS["tile"], LISTS["segment"]


def problem(batch, heads_q, heads_kv, seq_len, head_dim, dtype, seg_len, tile_m=128,
            tile_n=64, scale=None, causal=True, lists="tile", qperm=False, share_gqa=False) -> Problem:
    """dtype: torch.float32 / torch.bfloat16 (or 0 / 1).
    lists: "tile" (one list per query tile), "segment" (one list per segment), or
    "tile_blocks" / "segment_blocks" (the same with blocks of tile_n keys as entries).
    qperm: order the query rows of every segment by their guide score (Q_perm).
    share_gqa: one list per KV head, read by its query heads (S2O_SHARE_GQA)."""
    if isinstance(dtype, torch.dtype):
        dtype = {torch.float32: F32, torch.bfloat16: BF16}[dtype]
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    gran = LISTS[lists] | (QUERY_PERMUTATION if qperm else 0) | (SHARE_GQA if share_gqa else 0)
    return Problem(batch, heads_q, heads_kv, seq_len, head_dim, dtype, 1 if causal else 0,
                   seg_len, tile_m, tile_n, float(scale), gran)


def problem_for(q: torch.Tensor, k: torch.Tensor, seg_len: int, tile=(128, 64), scale=None,
                causal=True, lists="tile", qperm=False, share_gqa=False) -> Problem:
    B, Hq, N, d = q.shape
    return problem(B, Hq, k.shape[1], N, d, q.dtype, seg_len, tile[0], tile[1], scale, causal,
                   lists, qperm, share_gqa)


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: Optional[torch.Tensor], name: str, dtype=None) -> ctypes.c_void_p:
    if t is None:
        return ctypes.c_void_p(0)
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr() if t.numel() > 0 else 0)


def _tdtype(p: Problem):
    return torch.float32 if p.dtype == F32 else torch.bfloat16


def check_problem(p: Problem) -> int:
    return lib().s2o_check_problem(ctypes.byref(p))


def list_entries(p: Problem) -> int:
    n = lib().s2o_list_entries(ctypes.byref(p))
    if n < 0:
        _raise("s2o_list_entries", check_problem(p))
    return n


def list_offset(p: Problem, b: int, h: int, t: int) -> int:
    return lib().s2o_list_offset(ctypes.byref(p), b, h, t)


def score_workspace_bytes(p: Problem) -> int:
    return lib().s2o_score_workspace_bytes(ctypes.byref(p))


def build_index_workspace_bytes(p: Problem) -> int:
    return lib().s2o_build_index_workspace_bytes(ctypes.byref(p))


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def s2o_score(p: Problem, q: torch.Tensor, k: torch.Tensor, scores: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp32 importance scores of every list entry (history keys or blocks), in the list layout."""
    dt = _tdtype(p)
    n = list_entries(p)
    if scores is None:
        scores = torch.empty(n, dtype=torch.float32, device=q.device)
    wsb = score_workspace_bytes(p)
    if workspace is None:
        workspace = _workspace(wsb, q.device)
    st = lib().s2o_score(ctypes.byref(p), _dev(q, "q", dt), _dev(k, "k", dt),
                         _dev(scores, "scores", torch.float32), _dev(workspace, "workspace"),
                         workspace.numel(), _stream())
    _raise("s2o_score", st)
    return scores


# bytes of the static workspace s2o_score_noalloc uses (S2O_SCORE_NOALLOC_MAX_WORKSPACE)
SCORE_NOALLOC_MAX_WORKSPACE = 64 << 20


def s2o_score_noalloc(p: Problem, q: torch.Tensor, k: torch.Tensor,
                      scores: Optional[torch.Tensor] = None) -> torch.Tensor:
    """s2o_score with the library's static workspace (no caller workspace)."""
    dt = _tdtype(p)
    if scores is None:
        scores = torch.empty(list_entries(p), dtype=torch.float32, device=q.device)
    st = lib().s2o_score_noalloc(ctypes.byref(p), _dev(q, "q", dt), _dev(k, "k", dt),
                                 _dev(scores, "scores", torch.float32), _stream())
    _raise("s2o_score_noalloc", st)
    return scores


def s2o_build_index(p: Problem, scores: torch.Tensor, idx: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Index lists (keys or blocks), score descending, ties to the lower position."""
    n = list_entries(p)
    if idx is None:
        idx = torch.empty(n, dtype=torch.int32, device=scores.device)
    wsb = build_index_workspace_bytes(p)
    if workspace is None:
        workspace = _workspace(wsb, scores.device)
    st = lib().s2o_build_index(ctypes.byref(p), _dev(scores, "scores", torch.float32),
                               _dev(idx, "idx", torch.int32), _dev(workspace, "workspace"),
                               workspace.numel(), _stream())
    _raise("s2o_build_index", st)
    return idx


def s2o_attn_fwd(p: Problem, q, k, v, idx, tau: float, out=None, exec_tiles=None,
                 want_exec: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Gathered attention with early stop; returns (O, exec_tiles)."""
    dt = _tdtype(p)
    if out is None:
        out = torch.empty_like(q)
    if exec_tiles is None and want_exec:
        exec_tiles = torch.empty((p.batch, p.heads_q, p.seq_len // p.tile_m), dtype=torch.int32,
                                 device=q.device)
    st = lib().s2o_attn_fwd(ctypes.byref(p), _dev(q, "q", dt), _dev(k, "k", dt), _dev(v, "v", dt),
                            _dev(idx, "idx", torch.int32), float(tau), _dev(out, "out", dt),
                            _dev(exec_tiles, "exec_tiles", torch.int32), _stream())
    _raise("s2o_attn_fwd", st)
    return out, exec_tiles


def dense_attn_fwd(p: Problem, q, k, v, out=None) -> torch.Tensor:
    """Dense (FlashAttention-style) softmax attention with the same tiles."""
    dt = _tdtype(p)
    if out is None:
        out = torch.empty_like(q)
    st = lib().dense_attn_fwd(ctypes.byref(p), _dev(q, "q", dt), _dev(k, "k", dt), _dev(v, "v", dt),
                              _dev(out, "out", dt), _stream())
    _raise("dense_attn_fwd", st)
    return out


def s2o_attention(q, k, v, tau: float, seg_len: int, tile=(128, 64), scale=None, lists="tile",
                  qperm=False, share_gqa=False):
    """Whole path: score -> build_index -> attention.  Returns (O, exec_tiles)."""
    p = problem_for(q, k, seg_len, tile, scale, lists=lists, qperm=qperm, share_gqa=share_gqa)
    scores = s2o_score(p, q, k)
    idx = s2o_build_index(p, scores)
    return s2o_attn_fwd(p, q, k, v, idx, tau)
