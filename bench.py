"""Benchmark: S2O attention ms per layer at 128K tokens, Llama-3.1-8B head shape.

One step = the whole path for one attention layer (32 query heads, 8 KV
heads, d = 128, bf16, N = 131072, tiles 128x64, segments of 8192 tokens):
s2o_score -> s2o_build_index -> s2o_attn_fwd, on seeded synthetic inputs that
are resident in HBM before timing starts.

Before timing, tau is chosen as the largest value of a fixed sweep whose
output stays within an MSE of 1e-5 against this library's dense_attn_fwd
(mean over all B*Hq*N*d elements, fp32), then refined by a few geometric
bisection steps between it and the next sweep value (whose MSE is above the
budget); --tau skips both.  The same run also reports the speedup at the
stricter reading of the budget (MSE / mean(O_dense^2) <= 1e-5).

The headline uses one index list per query tile.  The same measurement is
repeated for the other list forms (per segment, blocks of 64 keys, Q_perm,
lists shared by the query heads of a KV head) and for the other workloads
(16K with its own tau sweep, 64K at tau = 1e-3, near-uniform 128K at tau = 0
and 1e-3), each as one compact row.

After the timed steps, the CPU leg runs the oracle on a fixed sample of the
headline workload (heads 0, 9, 18, 27 at the first and last tile of every
segment, plus 16 seeded (head, tile) pairs): its time, extrapolated to the
layer, is cpu_baseline; the GPU's lists, executed-tile counts and outputs on
the same tiles, and sampled rows of the dense kernel, are compared with it
("parity").  The ranking study measures on the same sample how well each list
form's order matches every row's true attention order.

stdout: one JSON line (under 4000 characters) with the fields the driver
parses; the full record (tau sweeps, the whole ranking study) is printed to
stderr as one line starting with "[bench] detail ".
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import threading
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "S2O attn ms/layer @128K Llama-3.1-8B shape; MFMA % on executed tiles"
MSE_BUDGET = 1e-5
BF16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
HBM_PEAK_GBS = 8000.0
RECORD_LIMIT = 4000              # characters of the stdout record
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_s2o_attn_fwd_llama8b_n128k.json")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters_attn_fwd_llama8b_n128k.json")
# the attention kernel's sources: its file and the shared geometry header it compiles
ATTN_SOURCE = [os.path.join(ROOT, "long_context_prefill_amd", "csrc", f) for f in ("attn_fwd.hip", "s2o_internal.h")]
STUDY_TAUS = (1e-2, 3e-3, 1e-3)  # ranking-study points reported beside tau*
FORM_NAMES = {"tile": "tile", "segment": "segment", "tile_blocks": "blocks", "segment_blocks": "seg_blocks",
              "tile+qperm": "qperm", "segment+qperm": "seg_qperm", "tile+gqa": "shared",
              "segment+gqa": "seg_shared"}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b_n128k")
    ap.add_argument("--tau", type=float, default=None, help="skip the sweep and use this tau")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle leg (cpu_baseline and parity)")
    ap.add_argument("--dense-reps", type=int, default=3)
    ap.add_argument("--modes", default="segment,tile_blocks,tile+qperm,tile+gqa",
                    help="list forms measured besides the headline per-tile lists ('' for none)")
    ap.add_argument("--workloads", default="llama8b_n16k,llama8b_n64k,uniform_n128k",
                    help="other workloads measured after the headline ('' for none)")
    ap.add_argument("--extra-steps", type=int, default=5, help="timed steps of the other workloads")
    ap.add_argument("--no-ranking-study", action="store_true")
    ap.add_argument("--no-clocks", action="store_true",
                    help="skip sampling the GPU clock and power while the attention kernel repeats")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration for profiles)")
    ap.add_argument("--detail-out", default=None, help="also write the full record to this file")
    return ap.parse_args(argv)


# ----------------------------------------------------------- tau and sampling --

def refine_tau(sweep, evaluate, budget=MSE_BUDGET, steps=4):
    """Bisect (geometrically) between the largest sweep tau within `budget` and
    the smallest one above it.  `evaluate(tau)` returns a sweep record with an
    "mse" field; the records it makes are appended to `sweep` (marked
    "refined") and the largest tau found within budget is returned, or None
    when the sweep has no such bracket."""
    ok = [r["tau"] for r in sweep if r["mse"] <= budget]
    bad = [r["tau"] for r in sweep if r["mse"] > budget]
    if not ok:
        return None
    lo = max(ok)
    above = [t for t in bad if t > lo]
    if not above or lo <= 0.0:
        return lo
    hi = min(above)
    for _ in range(steps):
        mid = float(np.sqrt(lo * hi))
        r = evaluate(mid)
        r["refined"] = True
        sweep.append(r)
        if r["mse"] <= budget:
            lo = mid
        else:
            hi = mid
    return lo


def stop_fired_share(exec_tiles, N, BM, BN, S):
    """Share of tiles with history whose early stop fired, i.e. that executed
    fewer pass-2 chunks than their list holds (exec_tiles [B, H, T]; pass 1 of
    tile t is ((t+1)*BM - a_t) / BN key tiles, its list a_t / BN chunks, for
    key and for block lists alike; not defined with Q_perm, whose pass 1
    depends on the row order)."""
    T = N // BM
    t = np.arange(T)
    a = (t * BM // S) * S
    n1 = ((t + 1) * BM - a) // BN
    full = n1 + a // BN
    has = a > 0
    if not has.any():
        return None
    ex = np.asarray(exec_tiles).reshape(-1, T)
    return float((ex[:, has] < full[has]).mean())


def sample_tiles(w, heads=(0, 9, 18, 27), n_random=16, seed=2026):
    """The measurement sample: for the given heads the first and last tile of
    every segment, plus n_random seeded (b, h, t) triples; sorted, no repeats."""
    T = w.N // w.tile_m
    P = w.seg_len // w.tile_m
    tiles = set()
    for h in heads:
        if h >= w.Hq:
            continue
        for s in range((T + P - 1) // P):
            tiles.add((0, h, s * P))
            tiles.add((0, h, min(T, (s + 1) * P) - 1))
    rng = np.random.default_rng(seed)
    for _ in range(n_random):
        tiles.add((int(rng.integers(w.B)), int(rng.integers(w.Hq)), int(rng.integers(T))))
    return sorted(tiles)


# ---------------------------------------------------- profiles and clocks -----

def source_hash(paths):
    """First 16 hex digits of the SHA-256 of the files' contents, concatenated in order."""
    h = hashlib.sha256()
    for path in paths:
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def traffic_record():
    """The committed traffic record of the attention kernel, or None when it is
    absent or was taken on a different version of the kernel's sources."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != source_hash(ATTN_SOURCE):
        return None
    return rec


def traffic_figure():
    """Bytes per launch beyond L2 (FETCH_SIZE + WRITE_SIZE, calibrated) from the
    committed record of this kernel source, or None."""
    rec = traffic_record()
    return rec.get("hbm_bytes_per_launch") if rec else None


def mfma_busy_counter():
    """Share of SIMD cycles the matrix cores were busy in the S2O attention
    kernel (SQ_VALU_MFMA_BUSY_CYCLES over SQ_BUSY_CYCLES scaled to SIMDs), from
    the committed counter profile of this kernel source; None otherwise."""
    try:
        rec = json.load(open(COUNTERS_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != source_hash(ATTN_SOURCE):
        return None
    k = rec.get("kernels", {}).get("s2o_attn_fwd (S2O schedule)")
    return round(k["mfma_busy"], 4) if k else None


def gather_figure(attn_ms):
    """The attention kernel's memory traffic per launch (committed counter
    record of this kernel source) over its live average duration:
      beyond_l2   FETCH_SIZE + WRITE_SIZE, every request that leaves L2
                  (Infinity Cache hits included), against the HBM peak;
      dram        TCC_EA0_RDREQ_DRAM / TCC_EA0_WRREQ_DRAM requests (64 B, or
                  32 B for the _32B read counter), when the record has them;
      l2_hit      TCC_HIT / (TCC_HIT + TCC_MISS), when the record has them.
    None without a matching record."""
    rec = traffic_record()
    if rec is None:
        return None
    s = attn_ms * 1e-3
    t = rec["hbm_bytes_per_launch"]
    out = {"beyond_l2_gbs": round(t / s / 1e9, 1), "beyond_l2_frac": round(t / s / 1e9 / HBM_PEAK_GBS, 4),
           "bytes_beyond_l2": t}
    if rec.get("dram_bytes_per_launch") is not None:
        d = rec["dram_bytes_per_launch"]
        out.update({"dram_gbs": round(d / s / 1e9, 1), "dram_frac": round(d / s / 1e9 / HBM_PEAK_GBS, 4),
                    "bytes_dram": d})
    if rec.get("l2_hit_rate") is not None:
        out["l2_hit"] = round(rec["l2_hit_rate"], 4)
    return out


def amd_smi_sample():
    """One reading: mean gfx clock over the XCDs (MHz) and socket power (W), or None."""
    try:
        r = subprocess.run(["amd-smi", "metric", "-c", "-p", "--json"], capture_output=True, text=True,
                           timeout=30)
        g = json.loads(r.stdout)["gpu_data"][0]
        clks = [float(v["clk"]["value"]) for k, v in g["clock"].items() if k.startswith("gfx_")]
        return sum(clks) / len(clks), float(g["power"]["socket_power"]["value"])
    except Exception:  # tool missing, busy or in another format: no reading
        return None


def clocks_under_load(launch, seconds=6.0):
    """Samples amd-smi from a second thread while `launch()` (one kernel launch)
    repeats on the GPU for about `seconds`, after the timed steps.  None when no
    reading was possible (or when run under a profiler, whose preload every
    child process would inherit)."""
    if "rocprof" in os.environ.get("LD_PRELOAD", ""):
        return None
    import torch
    samples, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            s = amd_smi_sample()
            if s is None:
                return
            samples.append(s)

    for _ in range(3):  # reach a steady clock first
        launch()
    torch.cuda.synchronize()
    th = threading.Thread(target=poll, daemon=True)
    th.start()
    t0 = time.time()
    while time.time() - t0 < seconds and th.is_alive():
        launch()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=60)
    if not samples:
        return None
    clk, pw = [c for c, _ in samples], [w for _, w in samples]
    return {"gfx_mhz_mean": round(sum(clk) / len(clk)), "gfx_mhz_min": round(min(clk)),
            "gfx_mhz_max": round(max(clk)), "socket_power_w_mean": round(sum(pw) / len(pw)),
            "socket_power_w_max": round(max(pw)), "samples": len(samples),
            "source": "amd-smi metric -c -p while s2o_attn_fwd repeats (headline lists and tau), "
                      "after the timed steps"}


# ------------------------------------------------------------ ranking study --

IMPORTANT_MASS = 0.9  # a row's important keys: the fewest history keys holding this share of its mass


def tile_truth(q, k, scale):
    """True attention order of query rows q [R, d] over history keys k [a, d]
    (fp32): logits, their exponentials against each row's max, every row's keys
    by descending logit, and the size of each row's important set (the fewest
    keys holding IMPORTANT_MASS of its history mass)."""
    xl = (q @ k.T) * np.float32(scale)                                  # [R, a]
    ex = np.exp(xl - xl.max(axis=1, keepdims=True))
    srt = np.argsort(-xl, axis=1, kind="stable")
    cum = np.cumsum(np.take_along_axis(ex, srt, 1), axis=1)
    m_i = (cum < IMPORTANT_MASS * cum[:, -1:]).sum(axis=1) + 1
    return {"xl": xl, "ex": ex, "srt": srt, "m_i": m_i}


def tile_metrics(tr, order, n_chunks, BN, chunks_by_tau=None):
    """Per-tile figures of one list order (key positions, the order the tile
    visits its history) with n_chunks pass-2 chunks executed, averaged over rows.
    E = the first n_chunks*BN keys of the order; for each row i:
      overlap   |E intersect top_i| / |E|, top_i = the |E| keys of largest logit
      mass      sum_{j in E} e^x_ij / sum_{j in top_i} e^x_ij  (1 = the best set of that size)
      coverage  sum_{j in E} e^x_ij / sum_{j < a} e^x_ij        (history mass executed)
      spearman  rank correlation between list position and -x_ij
    chunks_by_tau {tau: chunks}: with E_tau the keys executed at that tau and
    I_i row i's important set,
      precision |E_tau intersect I_i| / |E_tau| (None when E_tau is empty),
      recall    |E_tau intersect I_i| / |I_i|, and coverage as above."""
    xl, ex, srt, m_i = tr["xl"], tr["ex"], tr["srt"], tr["m_i"]
    R, a = xl.shape
    tot = ex.sum(axis=1)
    out = {}
    n = max(1, min(n_chunks * BN, a))
    E = order[:n]
    in_e = np.zeros(a, dtype=bool)
    in_e[E] = True
    top = srt[:, :n]
    out["overlap"] = float(in_e[top].mean())
    out["mass"] = float(np.mean(ex[:, E].sum(axis=1) / np.take_along_axis(ex, top, 1).sum(axis=1)))
    out["coverage"] = float(np.mean(ex[:, E].sum(axis=1) / tot))
    pos = np.empty(a, dtype=np.float64)
    pos[order] = np.arange(a)
    rk = np.empty(srt.shape, dtype=np.float64)                            # each key's true rank
    rk[np.arange(R)[:, None], srt] = np.arange(a, dtype=np.float64)[None, :]
    pc, rc = pos - pos.mean(), rk - rk.mean(axis=1, keepdims=True)
    out["spearman"] = float(np.mean((rc @ pc) / (np.sqrt((rc ** 2).sum(axis=1)) * np.sqrt((pc ** 2).sum()))))
    if chunks_by_tau:
        in_i = np.arange(a)[None, :] < m_i[:, None]                         # I_i in sorted coordinates
        out["by_tau"] = {}
        for tau, c in chunks_by_tau.items():
            nt = max(0, min(c * BN, a))
            e_t = np.zeros(a, dtype=bool)
            e_t[order[:nt]] = True
            hit = (e_t[srt] & in_i).sum(axis=1)
            out["by_tau"][tau] = {"precision": float(np.mean(hit / nt)) if nt else None,
                                  "recall": float(np.mean(hit / m_i)),
                                  "coverage": float(np.mean(ex[:, e_t].sum(axis=1) / tot))}
    return out


def expand_entries(entries, blocks, BN):
    """Key positions a list visits: the entries, or each block entry's BN keys."""
    e = np.asarray(entries, dtype=np.int64)
    return (e[:, None] * BN + np.arange(BN)).ravel() if blocks else e


def ranking_study(w, x, tiles, forms, threads=None):
    """Ranking accuracy of each list form on the sampled tiles.

    forms: {name: {"lists": {tile: entries}, "blocks": bool, "p1": {tile: pass-1 tiles},
                   "exec": {tau: {tile: executed tiles}}, "tau": tau*, "rows": {tile: rows} or None}}
    For every tile with history, tile_metrics at tau* (overlap, mass, coverage,
    spearman) and at every tau of "exec" (precision, recall, coverage), averaged
    over tiles (precision over tiles that executed a chunk); returned per form
    with "by_tau" in decreasing tau.  Plain numpy in fp32 from the stored inputs."""
    from long_context_prefill_amd import synth
    G = w.Hq // w.Hkv
    BN = w.tile_n
    widen = synth.f32_from_bf16_bits if w.dtype == "bf16" else (lambda z: np.asarray(z, np.float32))

    def one(tile):
        b, h, t = tile
        a = (t * w.tile_m // w.seg_len) * w.seg_len
        if a == 0:
            return tile, None
        k = widen(x["k"][b, h // G, :a])
        plain = None
        res = {}
        for name, f in forms.items():
            if f.get("rows"):
                tr = tile_truth(widen(x["q"][b, h, f["rows"][tile]]), k, w.scale)
            else:
                if plain is None:
                    plain = tile_truth(widen(x["q"][b, h, t * w.tile_m:(t + 1) * w.tile_m]), k, w.scale)
                tr = plain
            order = expand_entries(f["lists"][tile], f["blocks"], BN)
            p1 = f["p1"][tile]
            by = {tau: ex[tile] - p1 for tau, ex in f["exec"].items()}
            res[name] = tile_metrics(tr, order, by[f["tau"]], BN, by)
        return tile, res

    n_thr = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=n_thr) as pool:
        per_tile = [r for _, r in pool.map(one, tiles) if r is not None]
    out = {}
    for name, f in forms.items():
        rows = [r[name] for r in per_tile]
        s = {k: round(float(np.mean([r[k] for r in rows])), 4)
             for k in ("overlap", "mass", "coverage", "spearman")} | {"tiles": len(rows), "tau": f["tau"]}
        by = []
        for tau in sorted(f["exec"], reverse=True):
            vals = [r["by_tau"][tau] for r in rows]
            prec = [v["precision"] for v in vals if v["precision"] is not None]
            by.append({"tau": tau, "precision": round(float(np.mean(prec)), 4) if prec else None,
                       "recall": round(float(np.mean([v["recall"] for v in vals])), 4),
                       "coverage": round(float(np.mean([v["coverage"] for v in vals])), 4)})
        s["important_mass"] = IMPORTANT_MASS
        s["by_tau"] = by
        out[name] = s
    return out


def compact_study(study):
    """Per form, [precision, recall] (3 decimals) at tau* and at each of
    STUDY_TAUS, in that order (null where the sweep lacks the point)."""
    out = {}
    for name, s in study.items():
        pts = {e["tau"]: e for e in s["by_tau"]}
        row = []
        for tau in (s["tau"],) + STUDY_TAUS:
            e = pts.get(tau)
            row.append(None if e is None else [None if e["precision"] is None else round(e["precision"], 3),
                                               round(e["recall"], 3)])
        out[FORM_NAMES.get(name, name)] = row
    return out


# ------------------------------------------------------------ the GPU side --

class Workload:
    """One workload's inputs on the GPU, its dense output and the dense time."""

    def __init__(self, name, dense_reps):
        import torch

        import long_context_prefill_amd as s2o
        from long_context_prefill_amd import synth
        self.w = w = synth.WORKLOADS[name]
        log(f"generating {w.name} inputs")
        self.x = synth.make_inputs(w)
        dev = (lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)) \
            if w.dtype == "bf16" else (lambda a: torch.from_numpy(a).cuda())
        self.q, self.k, self.v = dev(self.x["q"]), dev(self.x["k"]), dev(self.x["v"])
        self.T = w.N // w.tile_m
        self.dense_tiles = sum(((t + 1) * w.tile_m) // w.tile_n for t in range(self.T)) * w.B * w.Hq
        self.flop_per_tile = 4.0 * w.tile_m * w.tile_n * w.d
        self.p_dense = self.problem()
        self.out_dense = torch.empty_like(self.q)
        s2o.dense_attn_fwd(self.p_dense, self.q, self.k, self.v, self.out_dense)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        ms = []
        for _ in range(dense_reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            s2o.dense_attn_fwd(self.p_dense, self.q, self.k, self.v, self.out_dense)
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        self.dense_ms = float(np.median(ms))
        log(f"[{w.name}] dense_attn_fwd {self.dense_ms:.2f} ms "
            f"({self.dense_tiles * self.flop_per_tile / self.dense_ms / 1e9:.0f} TFLOP/s)")
        self.dsq = float((self.out_dense.float() ** 2).mean())

    def problem(self, lists="tile", qperm=False, share=False):
        import long_context_prefill_amd as s2o
        w = self.w
        return s2o.problem(w.B, w.Hq, w.Hkv, w.N, w.d, 1 if w.dtype == "bf16" else 0, w.seg_len,
                           w.tile_m, w.tile_n, w.scale, lists=lists, qperm=qperm, share_gqa=share)


def measure(ctx, mode, taus, steps, warmup, refine=True, sample=(), after=None, clocks=False):
    """tau sweep (untimed), then `steps` timed steps of score -> build_index ->
    attention at the chosen tau.  mode: a list form ("tile", "segment",
    "tile_blocks", ...), "+qperm" for Q_perm, "+gqa" for lists shared by the
    query heads of a KV head.  sample: tiles whose lists and executed counts
    (at every tau) are kept for the ranking study.  after(p, idx, out,
    exec_tiles, tau): called after the timed steps, while the buffers live."""
    import torch

    import long_context_prefill_amd as s2o
    w, q, k, v = ctx.w, ctx.q, ctx.k, ctx.v
    lists, qperm, share = mode.split("+")[0], mode.endswith("+qperm"), mode.endswith("+gqa")
    p = ctx.problem(lists, qperm, share)
    n_list = s2o.list_entries(p)
    scores = torch.empty(max(n_list, 1), dtype=torch.float32, device="cuda")
    idx = torch.empty(max(n_list, 1), dtype=torch.int32, device="cuda")
    ws_score = torch.empty(max(s2o.score_workspace_bytes(p), 1), dtype=torch.uint8, device="cuda")
    ws_sort = torch.empty(max(s2o.build_index_workspace_bytes(p), 1), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    exec_tiles = torch.empty((w.B, w.Hq, ctx.T), dtype=torch.int32, device="cuda")
    s2o.s2o_score(p, q, k, scores, ws_score)
    s2o.s2o_build_index(p, scores, idx, ws_sort)
    sample_exec = {}
    tag = f"{w.name}/{mode}"

    def evaluate(tau):
        s2o.s2o_attn_fwd(p, q, k, v, idx, tau, out, exec_tiles)
        et = exec_tiles.cpu().numpy()
        sample_exec[tau] = {tl: int(et[tl]) for tl in sample}
        d = (out.float() - ctx.out_dense.float())
        mse = float((d ** 2).mean())
        max_abs = float(d.abs().max())
        density = float(et.sum()) / ctx.dense_tiles
        log(f"[{tag}] tau {tau:g}: density {density:.4f} mse {mse:.3e}")
        return {"tau": tau, "density": round(density, 4), "mse": mse, "rel_mse": mse / ctx.dsq,
                "max_abs_vs_dense": max_abs, "stop_fired": stop_fired_share(et, w.N, w.tile_m, w.tile_n, w.seg_len)
                if not qperm else None}

    sweep = [evaluate(tau) for tau in sorted(taus, reverse=True)]
    if refine and len(taus) > 1:
        refine_tau(sweep, evaluate)
    ok = [r for r in sweep if r["mse"] <= MSE_BUDGET]
    chosen = max(ok, key=lambda r: r["tau"]) if ok else min(sweep, key=lambda r: r["tau"])
    tau = chosen["tau"]
    stream = torch.cuda.current_stream()

    def timed(n, score_and_sort=True):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n)]
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for i in range(n):
            ev[i][0].record(stream)
            if score_and_sort:
                s2o.s2o_score(p, q, k, scores, ws_score)
            ev[i][1].record(stream)
            if score_and_sort:
                s2o.s2o_build_index(p, scores, idx, ws_sort)
            ev[i][2].record(stream)
            s2o.s2o_attn_fwd(p, q, k, v, idx, tau_t[0], out, exec_tiles)
            ev[i][3].record(stream)
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / n, np.array([[e[j].elapsed_time(e[j + 1]) for j in range(3)] for e in ev])

    tau_t = [tau]
    for _ in range(warmup):
        s2o.s2o_score(p, q, k, scores, ws_score)
        s2o.s2o_build_index(p, scores, idx, ws_sort)
        s2o.s2o_attn_fwd(p, q, k, v, idx, tau, out, exec_tiles)
    torch.cuda.synchronize()
    ms_per_step, ph = timed(steps)
    score_ms, sort_ms, attn_ms = (float(np.mean(ph[:, j])) for j in range(3))
    step = ph.sum(axis=1)
    step_stats = {"median": round(float(np.median(step)), 3), "min": round(float(step.min()), 3),
                  "p90": round(float(np.percentile(step, 90)), 3)}
    et = exec_tiles.cpu().numpy()
    executed = int(et.sum())
    res = {"mode": mode, "tau": tau, "ms_per_step": ms_per_step, "score_ms": score_ms, "sort_ms": sort_ms,
           "attn_ms": attn_ms, "step_stats": step_stats, "executed": executed,
           "density": executed / ctx.dense_tiles, "mse": chosen["mse"], "rel_mse": chosen["rel_mse"],
           "max_abs_vs_dense": chosen["max_abs_vs_dense"], "stop_fired": chosen["stop_fired"],
           "achieved": executed * ctx.flop_per_tile / (attn_ms * 1e-3) / 1e12, "sweep": sweep,
           "exec_tiles": et, "vs_dense": ctx.dense_ms / ms_per_step}
    # the stricter reading of the budget: MSE relative to the dense output's power
    ok_rel = [r for r in sweep if r["rel_mse"] <= MSE_BUDGET]
    if len(taus) > 1 and ok_rel:
        r_rel = max(ok_rel, key=lambda r: r["tau"])
        tau_t[0] = r_rel["tau"]
        _, ph_rel = timed(max(2, steps // 2), score_and_sort=False)
        attn_rel = float(np.mean(ph_rel[:, 2]))
        tau_t[0] = tau
        ms_rel = score_ms + sort_ms + attn_rel
        res["at_rel_mse_budget"] = {"tau": r_rel["tau"], "density": r_rel["density"], "rel_mse": r_rel["rel_mse"],
                                    "ms": ms_rel, "vs_dense": ctx.dense_ms / ms_rel}
        s2o.s2o_attn_fwd(p, q, k, v, idx, tau, out, exec_tiles)  # outputs at tau* again
    if clocks:
        log(f"[{tag}] sampling clocks and power while the attention kernel repeats")
        res["clocks"] = clocks_under_load(lambda: s2o.s2o_attn_fwd(p, q, k, v, idx, tau, out, exec_tiles))
    if sample:
        n_keys = n_list - (w.B * w.Hq * w.N if qperm else 0)
        rows, lists_h, p1 = {}, {}, {}
        for tl in sample:
            b, h, t = tl
            a = (t * w.tile_m // w.seg_len) * w.seg_len
            n_ent = a // w.tile_n if lists.endswith("blocks") else a
            off = s2o.list_offset(p, b, h, t)
            lists_h[tl] = idx[off:off + n_ent].cpu().numpy() if n_ent else np.zeros(0, np.int32)
            if qperm:
                o_ = n_keys + (b * w.Hq + h) * w.N + t * w.tile_m
                rows[tl] = a + idx[o_:o_ + w.tile_m].cpu().numpy().astype(np.int64)
                p1[tl] = (int(rows[tl].max()) + 1 - a + w.tile_n - 1) // w.tile_n
            else:
                p1[tl] = ((t + 1) * w.tile_m - a) // w.tile_n
        res["study_form"] = {"lists": lists_h, "blocks": lists.endswith("blocks"), "p1": p1,
                             "exec": sample_exec, "tau": tau, "rows": rows if qperm else None}
    if after is not None:
        after(p, idx, out, exec_tiles, tau)
    log(f"[{tag}] step {ms_per_step:.2f} ms = score {score_ms:.2f} + build_index {sort_ms:.2f} "
        f"+ attn {attn_ms:.2f} (dense {ctx.dense_ms:.2f})")
    del scores, idx, ws_score, ws_sort, out, exec_tiles
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------- the CPU leg -------

def host_cpu_model(path="/proc/cpuinfo"):
    """The host CPU's model name (first 'model name' line), or None."""
    try:
        with open(path) as f:
            for line in f:
                if line.startswith("model name"):
                    return " ".join(line.split(":", 1)[1].split())[:48]
    except OSError:
        pass
    return None


def cpu_leg(ctx, sample, tau, p, idx, out, exec_tiles, dense_rows_per_tile=4):
    """The oracle on the sample (pool, score, order, pass 1, pass 2 at tau) with
    all host threads: its time, scaled to the layer by executed keys, is the CPU
    baseline.  On the same tiles the GPU's lists, executed-tile counts and
    outputs are compared with it (tests/parity_util.compare: lists bit-exact,
    counts exact except near-tau ties, outputs within the bf16 tolerance), and
    dense_attn_fwd on dense_rows_per_tile rows of every sampled tile (first,
    last and seeded rows) with the oracle's dense rows."""
    import long_context_prefill_amd as s2o
    import oracle
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import parity_util
    w, x = ctx.w, ctx.x
    po = oracle.problem_from_workload(w)
    threads = oracle.num_threads()
    log(f"oracle on {len(sample)} sampled tiles ({threads} threads)")
    t0 = time.perf_counter()
    res = oracle.attn_tiles(po, x["q"], x["k"], x["v"], sample, tau, want_lists=True)
    dt = time.perf_counter() - t0

    class Lists:  # what parity_util.compare reads from a run: inputs, problems and the GPU's lists
        def tile_list(self, b, h, t):
            off = s2o.list_offset(p, b, h, t)
            return idx[off:off + oracle.list_len(po, t)].cpu().numpy()
    run = Lists()
    run.w, run.po, run.x = w, po, x
    rep = parity_util.compare(run, sample, tau, out, exec_tiles, check_lists=True, res=res)
    tol = parity_util.TOL[w.dtype]
    parity = {"tiles": rep["tiles"], "tau": tau, "list_mismatch": rep["list_mismatch"],
              "exec_mismatch": rep["exec_mismatch"], "near_tau": rep["near_tau"],
              "max_abs": rep["max_abs"], "mean_abs": rep["mean_abs"],
              "ok": bool(rep["list_mismatch"] == 0 and rep["exec_mismatch"] == 0 and rep["max_abs"] <= tol["max_abs"]
                         and (tol["mean_abs"] is None or rep["mean_abs"] <= tol["mean_abs"]))}
    rng = np.random.default_rng(99)
    req = []
    for b, h, t in sample:
        r0 = t * w.tile_m
        picks = {r0, r0 + w.tile_m - 1} | {int(r0 + rng.integers(w.tile_m)) for _ in range(dense_rows_per_tile - 2)}
        req += [(b, h, r, r + 1) for r in sorted(picks)]
    log(f"oracle dense rows: {len(req)}")
    ref = oracle.dense_requests(po, x["q"], x["k"], x["v"], req)
    od = ctx.out_dense
    dmax, dsum, dn = 0.0, 0.0, 0
    for (b, h, i0, i1), r in zip(req, ref):
        dd = np.abs(od[b, h, i0:i1].float().cpu().numpy().astype(np.float64) - r)
        dmax, dsum, dn = max(dmax, float(dd.max())), dsum + float(dd.sum()), dn + dd.size
    parity["dense_rows"] = len(req)
    parity["dense_max_abs"] = dmax
    parity["dense_mean_abs"] = dsum / max(dn, 1)
    parity["ok"] = parity["ok"] and dmax <= tol["max_abs"] and (tol["mean_abs"] is None or dsum / dn <= tol["mean_abs"])
    sample_keys = int(res["n_exec"].sum()) * w.tile_n
    layer_keys = int(exec_tiles.sum()) * w.tile_n
    cpu = {"value": round(dt * 1e3 * layer_keys / max(sample_keys, 1), 1), "unit": "ms", "cores": threads,
           "cpu": host_cpu_model(), "kind": "oracle", "extrapolated": True,
           "sample": (f"{len(sample)} tiles (heads 0,9,18,27: first+last of each segment; 16 seeded) at tau*, "
                      f"{dt:.1f} s, x executed keys {layer_keys}/{sample_keys}")}
    log(f"parity {parity}")
    return cpu, parity


# ----------------------------------------------------------------- record ----

def r3(x):
    return None if x is None else round(float(x), 3)


def sig(x, n=3):
    return None if x is None else float(f"{float(x):.{n}g}")


def r2(x):
    return None if x is None else round(float(x), 2)


def compact_form(r):
    return {"ms": r2(r["ms_per_step"]), "tau": sig(r["tau"]), "density": round(r["density"], 3),
            "mse": sig(r["mse"], 2), "phases": [r2(r["score_ms"]), r2(r["sort_ms"]), r2(r["attn_ms"])],
            "vs_dense": r3(r["vs_dense"])}


def compact_workload(ctx, rs):
    """One row per extra workload: dense time and, per tau measured, the S2O
    figures (with tau = 0, the largest output difference from dense)."""
    row = {"dense_ms": r2(ctx.dense_ms)}
    for r in rs:
        e = compact_form(r) | {"stop_fired": sig(r["stop_fired"], 2)}
        if r["tau"] == 0.0:
            e["max_abs_vs_dense"] = sig(r["max_abs_vs_dense"], 2)
        row[f"tau={sig(r['tau'])}"] = e
    return row


def build_record(args, w, main, dense_ms, forms, workloads, parity, cpu, study, traffic, busy):
    """The stdout record (compact) and the full record (the same plus sweeps and the study)."""
    rec = {
        "metric": METRIC, "value": r3(main["ms_per_step"]), "unit": "ms", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": r3(main["ms_per_step"]),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded; stripes, sinks and a local band per KV group)",
        "config": {"workload": w.name, "batch": w.B, "heads_q": w.Hq, "heads_kv": w.Hkv, "seq_len": w.N,
                   "head_dim": w.d, "tile": [w.tile_m, w.tile_n], "seg_len": w.seg_len,
                   "lists": "per query tile", "tau": main["tau"], "parallelism": "single GPU"},
        "phases_ms": {"s2o_score": r3(main["score_ms"]), "s2o_build_index": r3(main["sort_ms"]),
                      "s2o_attn_fwd": r3(main["attn_ms"])},
        "step_ms": main["step_stats"],
        "dense_attn_fwd_ms": r3(dense_ms),
        "speedup_vs_dense": r3(dense_ms / main["ms_per_step"]),
        "attn_speedup_vs_dense": r3(dense_ms / main["attn_ms"]),
        "density": round(main["density"], 4), "mse_vs_dense": sig(main["mse"]),
        "rel_mse_vs_dense": sig(main["rel_mse"]),
        "stop_fired_share": sig(main["stop_fired"]),
        "mfma_pct_executed_tiles": round(100.0 * main["achieved"] / BF16_MFMA_PEAK_TFLOPS, 2),
        "mfma_busy_counter": busy,
        "effective_tflops_executed_tiles": round(main["achieved"], 1),
        "roofline": {"bound": "mfma", "achieved": round(main["achieved"], 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(main["achieved"] / BF16_MFMA_PEAK_TFLOPS, 4),
                     "traffic": traffic, "kernel": "s2o_attn_fwd",
                     "work": f"{main['executed']} executed 128x64 tiles x 4.19 MFLOP"},
        "gathers": gather_figure(main["attn_ms"]),
    }
    if main.get("at_rel_mse_budget"):
        a = main["at_rel_mse_budget"]
        rec["at_rel_mse_1e-5"] = {"tau": sig(a["tau"]), "density": a["density"], "ms": r3(a["ms"]),
                                  "vs_dense": r3(a["vs_dense"])}
    c = main.get("clocks")
    if c:
        rec["clocks_during_attention"] = {"gfx_mhz": c["gfx_mhz_mean"], "power_w": c["socket_power_w_mean"],
                                          "samples": c["samples"]}
    if forms:
        rec["forms"] = {FORM_NAMES.get(m, m): compact_form(r) for m, r in forms.items()}
    if workloads:
        rec["workloads"] = workloads
    if parity is not None:
        rec["parity"] = {k: (sig(v) if isinstance(v, float) else v) for k, v in parity.items()}
    if study is not None:
        rec["ranking_study"] = {"tiles": next(iter(study.values()))["tiles"], "important_mass": IMPORTANT_MASS,
                                "taus": ["tau*"] + list(STUDY_TAUS), "precision_recall": compact_study(study)}
    if cpu is not None:
        rec["cpu_baseline"] = cpu
    full = dict(rec)
    full["tau_sweep"] = main["sweep"]
    if main.get("clocks"):
        full["clocks_during_attention"] = main["clocks"]
    if forms:
        full["form_sweeps"] = {m: r["sweep"] for m, r in forms.items()}
    if study is not None:
        full["ranking_study"] = study
    return rec, full


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the layer "
              "shards by KV head with no communication, so one GPU here runs all eight KV heads)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_calibration:
        # a plain copy of known size: 1 GiB read + 1 GiB written; its FETCH_SIZE and
        # WRITE_SIZE counters calibrate the attention kernel's traffic figures
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ctx = Workload(args.workload, args.dense_reps)
    w = ctx.w
    want_study = not args.no_ranking_study
    sample = sample_tiles(w)
    oracle_out = {}

    def after(p, idx, out, exec_tiles, tau):
        if not args.no_cpu_baseline:
            oracle_out["cpu"], oracle_out["parity"] = cpu_leg(ctx, sample, tau, p, idx, out, exec_tiles)

    taus = [args.tau] if args.tau is not None else list(w.taus)
    main_r = measure(ctx, "tile", taus, args.steps, args.warmup, sample=sample if want_study else (),
                     after=after, clocks=not args.no_clocks)
    forms = {}
    for m in [m for m in args.modes.split(",") if m]:
        forms[m] = measure(ctx, m, taus, args.steps, args.warmup, sample=sample if want_study else ())
    study = None
    if want_study:
        log(f"ranking study on {len(sample)} sampled tiles, {1 + len(forms)} list forms")
        sf = {"tile": main_r["study_form"]} | {m: r["study_form"] for m, r in forms.items()}
        study = ranking_study(w, ctx.x, sample, sf)
    dense_ms = ctx.dense_ms
    head = (w, main_r, dense_ms, forms, oracle_out.get("parity"), oracle_out.get("cpu"), study)
    del ctx
    torch.cuda.empty_cache()

    workloads = {}
    for name in [n for n in args.workloads.split(",") if n and n != w.name]:
        c = Workload(name, max(1, args.dense_reps - 1))
        wl = c.w
        if wl.structure == "uniform":   # tau = 0 must reproduce dense attention; tau = 1e-3: overhead case
            rs = [measure(c, "tile", [t], args.extra_steps, 1, refine=False) for t in wl.taus]
        else:                          # its own sweep and refinement (a fixed tau when it lists one)
            rs = [measure(c, "tile", list(wl.taus), args.extra_steps, 1, refine=len(wl.taus) > 1)]
        workloads[name] = compact_workload(c, rs)
        del c
        torch.cuda.empty_cache()

    w, main_r, dense_ms, forms, parity, cpu, study = head
    rec, full = build_record(args, w, main_r, dense_ms, forms, workloads, parity, cpu, study,
                             traffic_figure(), mfma_busy_counter())
    print("[bench] detail " + json.dumps(full), file=sys.stderr, flush=True)
    if args.detail_out:
        with open(args.detail_out, "w") as f:
            json.dump(full, f, indent=1)
    line = json.dumps(rec, separators=(",", ":"))
    if len(line) > RECORD_LIMIT:
        log(f"record is {len(line)} characters (limit {RECORD_LIMIT})")
    print(line, flush=True)


if __name__ == "__main__":
    main()
