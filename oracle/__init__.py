"""CPU oracle for S2O causal-prefill attention -- test infrastructure only.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does, and
this package never imports the product.  The arithmetic lives in
``s2o_oracle.c`` (plain C, fp32 estimator in its canonical order, fp64
attention); this module only marshals numpy arrays through ctypes.

Parity status of each function (the pins live in ``tests/test_oracle_pins.py``):

* ``pool`` / ``score_tile``: pinned (exact special cases, fp64 error bound).
* ``pool_block`` and block lists: pinned (exact dyadic block means; block
  scores of block-constant keys equal the key scores, and their block order
  expands to the key order; tau = 0 equals dense attention; the Q = 0 closed
  form).
* ``order``: pinned (permutation, order, ties, independent Python sort).
* ``attn_tile`` / ``attn_tiles``: pinned (tau = 0 equals dense attention from
  torch's fp64 SDPA; Q = 0 closed form of the stop rule including the equality
  case; restricted-softmax identity; skipped-mass bounds).
* ``dense_rows``: pinned (torch fp64 SDPA and a numpy softmax).
* shared (GQA) lists: pinned (exact dyadic group means; every head of a group
  reads one list; G = 1 equals per-head lists; tau = 0 equals dense attention).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# S2O_ORACLE_LIB lets the mutation test load a deliberately broken copy
LIB_PATH = os.environ.get("S2O_ORACLE_LIB", os.path.join(_HERE, "libs2o_oracle.so"))
SOURCE = os.path.join(_HERE, "s2o_oracle.c")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2 -fopenmp -ffp-contract=off)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC",
               "-shared", SOURCE, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


class Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("N", ctypes.c_int32), ("d", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("seg_len", ctypes.c_int32), ("tile_m", ctypes.c_int32),
                ("tile_n", ctypes.c_int32), ("scale", ctypes.c_double),
                ("per_segment", ctypes.c_int32), ("block_lists", ctypes.c_int32),
                ("qperm", ctypes.c_int32), ("share_gqa", ctypes.c_int32)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(Problem)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        sig = {
            "oracle_num_tiles": (i32, [P]),
            "oracle_seg_start": (i64, [P, ctypes.c_int]),
            "oracle_pass1_tiles": (i32, [P, ctypes.c_int]),
            "oracle_list_offset": (i64, [P, ctypes.c_int, ctypes.c_int, ctypes.c_int]),
            "oracle_list_entries": (i64, [P]),
            "oracle_list_len": (i64, [P, ctypes.c_int]),
            "oracle_pool_block": (None, [P, vp, ctypes.c_int, ctypes.c_int, i64, vp]),
            "oracle_pool": (None, [P, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]),
            "oracle_rep_query": (None, [P, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]),
            "oracle_guide": (None, [P, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]),
            "oracle_query_scores": (None, [P, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]),
            "oracle_tile_rows": (None, [P, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]),
            "oracle_query_list_offset": (i64, [P, ctypes.c_int, ctypes.c_int, ctypes.c_int]),
            "oracle_score_tile": (None, [P, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]),
            "oracle_order": (None, [vp, i64, vp]),
            "oracle_attn_tile": (i32, [P, vp, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       vp, dbl, i32, vp, vp, vp]),
            "oracle_dense_rows": (None, [P, vp, vp, vp, ctypes.c_int, ctypes.c_int, i64, i64, vp]),
            "oracle_num_threads": (ctypes.c_int, []),
            "oracle_scores_all": (None, [P, vp, vp, vp]),
            "oracle_lists_all": (None, [P, vp, vp]),
            "oracle_attn_tiles": (None, [P, vp, vp, vp, vp, i64, vp, dbl, vp, vp, vp, vp, vp,
                                         i64, vp, i64]),
            "oracle_dense_requests": (None, [P, vp, vp, vp, vp, i64, vp, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def problem(B, Hq, Hkv, N, d, dtype, seg_len, tile_m, tile_n, scale, per_segment=False,
            block_lists=False, qperm=False, share_gqa=False) -> Problem:
    """dtype: "f32" (float32 arrays) or "bf16" (uint16 bit-pattern arrays).
    per_segment: one list per segment (shared by its tiles) instead of per tile.
    block_lists: list entries are blocks of tile_n keys instead of keys.
    qperm: query rows ordered within each segment by a guide score (Q_perm).
    share_gqa: one list per KV head, shared by its query heads (not with qperm)."""
    if qperm and share_gqa:
        raise ValueError("shared lists are not defined with the query permutation")
    return Problem(B, Hq, Hkv, N, d, 0 if dtype == "f32" else 1, seg_len, tile_m, tile_n,
                   float(scale), 1 if per_segment else 0, 1 if block_lists else 0, 1 if qperm else 0,
                   1 if share_gqa else 0)


def problem_from_workload(w, seg_len=None, per_segment=False, block_lists=False,
                          qperm=False, share_gqa=False) -> Problem:
    return problem(w.B, w.Hq, w.Hkv, w.N, w.d, w.dtype,
                   w.seg_len if seg_len is None else seg_len, w.tile_m, w.tile_n, w.scale,
                   per_segment, block_lists, qperm, share_gqa)


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _check(a, p: Problem, name):
    want = np.float32 if p.dtype == 0 else np.uint16
    if a.dtype != want or not a.flags.c_contiguous:
        raise TypeError(f"{name}: expected contiguous {want.__name__} array")
    return a


def num_tiles(p):
    return _load().oracle_num_tiles(ctypes.byref(p))


def seg_start(p, t):
    return _load().oracle_seg_start(ctypes.byref(p), t)


def pass1_tiles(p, t):
    return _load().oracle_pass1_tiles(ctypes.byref(p), t)


def list_offset(p, b, h, t):
    return _load().oracle_list_offset(ctypes.byref(p), b, h, t)


def list_entries(p):
    return _load().oracle_list_entries(ctypes.byref(p))


def list_len(p, t):
    """Entries of the list tile t uses (keys, or blocks of tile_n keys)."""
    return _load().oracle_list_len(ctypes.byref(p), t)


def pool_block(p, K, b, g, c):
    """Mean key of block c of KV head g."""
    out = np.empty(p.d, dtype=np.float32)
    _load().oracle_pool_block(ctypes.byref(p), _ptr(_check(K, p, "K")), b, g, c, _ptr(out))
    return out


def num_threads():
    return _load().oracle_num_threads()


def _kptr(p, K):
    if K is None:
        if p.qperm:
            raise ValueError("Q_perm needs K (the segment guide is the mean key)")
        return None
    return _ptr(_check(K, p, "K"))


def pool(p, Q, b, h, t, K=None):
    out = np.empty(p.d, dtype=np.float32)
    _load().oracle_pool(ctypes.byref(p), _ptr(_check(Q, p, "Q")), _kptr(p, K), b, h, t, _ptr(out))
    return out


def rep_query(p, Q, b, h, t, K=None):
    """The representative query of the list tile t uses (tile mean or segment mean)."""
    out = np.empty(p.d, dtype=np.float32)
    _load().oracle_rep_query(ctypes.byref(p), _ptr(_check(Q, p, "Q")), _kptr(p, K), b, h, t, _ptr(out))
    return out


def guide(p, K, b, g, s):
    """Q_perm guide of segment s for KV head g (the segment's mean key)."""
    out = np.empty(p.d, dtype=np.float32)
    _load().oracle_guide(ctypes.byref(p), _ptr(_check(K, p, "K")), b, g, s, _ptr(out))
    return out


def query_scores(p, Q, K, b, h, s):
    """Q_perm importance scores of the rows of segment s, in row order."""
    a = s * p.seg_len
    n = min(p.N, a + p.seg_len) - a
    out = np.empty(n, dtype=np.float32)
    _load().oracle_query_scores(ctypes.byref(p), _ptr(_check(Q, p, "Q")), _ptr(_check(K, p, "K")),
                                b, h, s, _ptr(out))
    return out


def tile_rows(p, Q, K, b, h, t):
    """Absolute rows of query tile t, in tile order."""
    out = np.empty(p.tile_m, dtype=np.int64)
    _load().oracle_tile_rows(ctypes.byref(p), _ptr(_check(Q, p, "Q")), _kptr(p, K), b, h, t, _ptr(out))
    return out


def query_list_offset(p, b, h, s):
    return _load().oracle_query_list_offset(ctypes.byref(p), b, h, s)


def score_tile(p, Q, K, b, h, t):
    a = list_len(p, t)
    out = np.empty(max(a, 1), dtype=np.float32)
    _load().oracle_score_tile(ctypes.byref(p), _ptr(_check(Q, p, "Q")), _ptr(_check(K, p, "K")),
                              b, h, t, _ptr(out))
    return out[:a]


def order(scores):
    s = np.ascontiguousarray(scores, dtype=np.float32)
    out = np.empty(max(len(s), 1), dtype=np.int32)
    _load().oracle_order(_ptr(s), len(s), _ptr(out))
    return out[:len(s)]


def attn_tile(p, Q, K, V, b, h, t, lst, tau, force_n=0):
    """Returns (out [BM, d] float64, n_exec, chunks executed, gstar per chunk)."""
    lib = _load()
    a = list_len(p, t)
    lst = np.ascontiguousarray(lst, dtype=np.int32)
    if len(lst) != a:
        raise ValueError("list length must equal the tile's list length")
    out = np.empty((p.tile_m, p.d), dtype=np.float64)
    n_exec = ctypes.c_int32()
    gstar = np.zeros(max(seg_start(p, t) // p.tile_n, 1), dtype=np.float64)
    buf = lst if a > 0 else np.zeros(1, dtype=np.int32)
    c = lib.oracle_attn_tile(ctypes.byref(p), _ptr(_check(Q, p, "Q")), _ptr(_check(K, p, "K")),
                             _ptr(_check(V, p, "V")), b, h, t, _ptr(buf), float(tau),
                             int(force_n), _ptr(out), ctypes.byref(n_exec), _ptr(gstar))
    return out, n_exec.value, c, gstar[:c]


def attn_tiles(p, Q, K, V, tiles, tau, lists=None, force_n=None, want_lists=False):
    """Run a set of tiles [(b, h, t), ...] in parallel.

    Returns dict: out [n, BM, d] float64, n_exec [n], chunks [n],
    gstar [n, max_chunks] (valid up to chunks[i]), lists (if want_lists:
    [n, max_list] int32, valid up to the tile's history length).
    """
    lib = _load()
    tiles = np.ascontiguousarray(np.asarray(tiles, dtype=np.int32).reshape(-1, 3))
    n = len(tiles)
    max_list = max([list_len(p, int(t)) for _, _, t in tiles] + [1])
    max_chunks = max(max([seg_start(p, int(t)) for _, _, t in tiles] + [1]) // p.tile_n, 1)
    out = np.empty((n, p.tile_m, p.d), dtype=np.float64)
    n_exec = np.empty(n, dtype=np.int32)
    chunks = np.empty(n, dtype=np.int32)
    gstar = np.zeros((n, max_chunks), dtype=np.float64)
    lout = np.empty((n, max_list), dtype=np.int32) if want_lists else None
    fn = None if force_n is None else np.ascontiguousarray(force_n, dtype=np.int32)
    if lists is not None:
        lists = np.ascontiguousarray(lists, dtype=np.int32)
    lib.oracle_attn_tiles(ctypes.byref(p), _ptr(_check(Q, p, "Q")), _ptr(_check(K, p, "K")),
                          _ptr(_check(V, p, "V")), _ptr(tiles), n, _ptr(lists), float(tau),
                          _ptr(fn), _ptr(out), _ptr(n_exec), _ptr(chunks), _ptr(gstar),
                          max_chunks, _ptr(lout), max_list)
    res = {"out": out, "n_exec": n_exec, "chunks": chunks, "gstar": gstar,
           "rows": np.stack([tile_rows(p, Q, K, int(b), int(h), int(t)) for b, h, t in tiles])
           if p.qperm else None}
    if want_lists:
        res["lists"] = lout
    return res


def dense_rows(p, Q, K, V, b, h, i0, i1):
    out = np.empty((i1 - i0, p.d), dtype=np.float64)
    _load().oracle_dense_rows(ctypes.byref(p), _ptr(_check(Q, p, "Q")), _ptr(_check(K, p, "K")),
                              _ptr(_check(V, p, "V")), b, h, i0, i1, _ptr(out))
    return out


def dense_requests(p, Q, K, V, requests):
    """requests: [(b, h, i0, i1), ...] -> list of float64 [i1-i0, d] arrays."""
    req = np.ascontiguousarray(np.asarray(requests, dtype=np.int64).reshape(-1, 4))
    rows = req[:, 3] - req[:, 2]
    offs = np.concatenate([[0], np.cumsum(rows * p.d)[:-1]]).astype(np.int64)
    out = np.empty(int(rows.sum()) * p.d, dtype=np.float64)
    _load().oracle_dense_requests(ctypes.byref(p), _ptr(_check(Q, p, "Q")),
                                  _ptr(_check(K, p, "K")), _ptr(_check(V, p, "V")), _ptr(req),
                                  len(req), _ptr(offs), _ptr(out))
    return [out[o:o + r * p.d].reshape(r, p.d) for o, r in zip(offs, rows)]


def scores_all(p, Q, K):
    out = np.empty(max(list_entries(p), 1), dtype=np.float32)
    _load().oracle_scores_all(ctypes.byref(p), _ptr(_check(Q, p, "Q")), _ptr(_check(K, p, "K")),
                              _ptr(out))
    return out[:list_entries(p)]


def lists_all(p, scores):
    s = np.ascontiguousarray(scores, dtype=np.float32)
    out = np.empty(max(len(s), 1), dtype=np.int32)
    _load().oracle_lists_all(ctypes.byref(p), _ptr(s if len(s) else np.zeros(1, np.float32)),
                             _ptr(out))
    return out[:len(s)]
