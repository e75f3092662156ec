"""Shared helpers for the GPU parity tests: move seeded inputs to the device,
run the HIP path through the C ABI, and compare against the CPU oracle.

Acceptance rules:
  * scores and index lists: bit-exact;
  * executed-tile counts: equal, except where the oracle's largest gain at the
    chunk where the two diverge lies within 1e-4 relative of tau (floating
    point decides the stop there); such tiles are counted, and their outputs
    are re-checked against the oracle forced to the GPU's chunk count;
  * outputs: fp32 max-abs <= 1e-4; bf16 max-abs <= 2e-2 and mean-abs <= 2e-3.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

import long_context_prefill_amd as s2o
import oracle
from long_context_prefill_amd import synth

NEAR_TAU_REL = 1e-4
TOL = {"f32": dict(max_abs=1e-4, mean_abs=None), "bf16": dict(max_abs=2e-2, mean_abs=2e-3)}


def say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def to_device(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(x).cuda()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def gpu_problem(w, seg_len=None, lists="tile", qperm=False, share_gqa=False):
    return s2o.problem(w.B, w.Hq, w.Hkv, w.N, w.d, 1 if w.dtype == "bf16" else 0,
                       w.seg_len if seg_len is None else seg_len, w.tile_m, w.tile_n, w.scale,
                       lists=lists, qperm=qperm, share_gqa=share_gqa)


class GpuRun:
    """Inputs on the device plus scores and lists from the HIP path."""

    def __init__(self, w, x, seg_len=None, lists="tile", qperm=False, share_gqa=False):
        self.w = w
        self.lists = lists
        self.p = gpu_problem(w, seg_len, lists, qperm, share_gqa)
        self.po = oracle.problem_from_workload(w, seg_len, per_segment=lists.startswith("segment"),
                                               block_lists=lists.endswith("blocks"), qperm=qperm,
                                               share_gqa=share_gqa)
        self.x = x
        self.q, self.k, self.v = (to_device(x[n]) for n in ("q", "k", "v"))
        say(f"{w.name}: score + build_index ({lists} lists{', shared' if share_gqa else ''}, "
            f"{s2o.list_entries(self.p)} entries)")
        self.scores = s2o.s2o_score(self.p, self.q, self.k)
        self.idx = s2o.s2o_build_index(self.p, self.scores)
        torch.cuda.synchronize()

    def attn(self, tau):
        say(f"{self.w.name}: s2o_attn_fwd tau={tau}")
        o, ex = s2o.s2o_attn_fwd(self.p, self.q, self.k, self.v, self.idx, tau)
        torch.cuda.synchronize()
        return o, ex

    def dense(self):
        say(f"{self.w.name}: dense_attn_fwd")
        o = s2o.dense_attn_fwd(self.p, self.q, self.k, self.v)
        torch.cuda.synchronize()
        return o

    def tile_list(self, b, h, t):
        off = s2o.list_offset(self.p, b, h, t)
        a = oracle.list_len(self.po, t)
        return self.idx[off:off + a].cpu().numpy()

    def tile_scores(self, b, h, t):
        off = s2o.list_offset(self.p, b, h, t)
        a = oracle.list_len(self.po, t)
        return self.scores[off:off + a].cpu().numpy()


def sample_tiles(w, heads, n_random, seed, seg_len=None):
    """First and last tile of every segment for the given heads, plus random tiles."""
    S = w.seg_len if seg_len is None else seg_len
    T = w.N // w.tile_m
    P = S // w.tile_m
    tiles = set()
    for h in heads:
        for s in range((T + P - 1) // P):
            tiles.add((0, h, s * P))
            tiles.add((0, h, min(T, (s + 1) * P) - 1))
    rng = np.random.default_rng(seed)
    for _ in range(n_random):
        tiles.add((int(rng.integers(w.B)), int(rng.integers(w.Hq)), int(rng.integers(T))))
    return sorted(tiles)


def compare(run: GpuRun, tiles, tau, o_gpu, ex_gpu, check_lists=True, res=None):
    """Compare the given tiles against the oracle; returns a report dict.
    res: the oracle's result for these tiles (attn_tiles with want_lists=True),
    computed here when not given."""
    w, po = run.w, run.po
    BM = w.tile_m
    if res is None:
        res = oracle.attn_tiles(po, run.x["q"], run.x["k"], run.x["v"], tiles, tau, want_lists=True)
    ex = ex_gpu.cpu().numpy()
    rep = dict(tiles=len(tiles), near_tau=0, list_mismatch=0, exec_mismatch=0, max_abs=0.0,
               sum_abs=0.0, n=0)
    forced = []
    for n, (b, h, t) in enumerate(tiles):
        a = oracle.list_len(po, t)
        if check_lists and a > 0:
            if not np.array_equal(run.tile_list(b, h, t), res["lists"][n, :a]):
                rep["list_mismatch"] += 1
        ng, no = int(ex[b, h, t]), int(res["n_exec"][n])
        if ng != no:
            p1 = int(res["n_exec"][n]) - int(res["chunks"][n])
            c = min(ng, no) - p1 - 1
            g = res["gstar"][n, c] if c >= 0 else -1.0
            if c >= 0 and abs(g - tau) <= NEAR_TAU_REL * tau:
                rep["near_tau"] += 1
                forced.append((n, (b, h, t), ng - p1))
            else:
                rep["exec_mismatch"] += 1
                say(f"exec mismatch at {(b, h, t)}: gpu {ng} oracle {no} (gain {g}, tau {tau})")
            continue
        rows = res["rows"][n] if res["rows"] is not None else np.arange(t * BM, (t + 1) * BM)
        og = f64(o_gpu[b, h][torch.as_tensor(rows, device=o_gpu.device)])
        d = np.abs(og - res["out"][n])
        rep["max_abs"] = max(rep["max_abs"], float(d.max()))
        rep["sum_abs"] += float(d.sum())
        rep["n"] += d.size
    if forced:
        fres = oracle.attn_tiles(po, run.x["q"], run.x["k"], run.x["v"], [f[1] for f in forced],
                                 tau, force_n=[f[2] for f in forced])
        for i, (_, (b, h, t), _) in enumerate(forced):
            rows = fres["rows"][i] if fres["rows"] is not None else np.arange(t * BM, (t + 1) * BM)
            og = f64(o_gpu[b, h][torch.as_tensor(rows, device=o_gpu.device)])
            d = np.abs(og - fres["out"][i])
            rep["max_abs"] = max(rep["max_abs"], float(d.max()))
            rep["sum_abs"] += float(d.sum())
            rep["n"] += d.size
    rep["mean_abs"] = rep["sum_abs"] / max(rep["n"], 1)
    return rep


def assert_report(rep, dtype):
    tol = TOL[dtype]
    say(f"report: {rep}")
    assert rep["list_mismatch"] == 0, rep
    assert rep["exec_mismatch"] == 0, rep
    assert rep["max_abs"] <= tol["max_abs"], rep
    if tol["mean_abs"] is not None:
        assert rep["mean_abs"] <= tol["mean_abs"], rep
