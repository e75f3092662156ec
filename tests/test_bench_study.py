"""CPU checks of the ranking study bench.py reports (no GPU): on inputs whose
true attention order is known, the study's figures take their extreme values."""

import numpy as np

import bench
from long_context_prefill_amd import synth


def _problem(N=512, d=16, BM=64, BN=64, S=256):
    w = synth.custom_workload(B=1, Hq=1, Hkv=1, N=N, d=d, dtype="f32", tile_m=BM, tile_n=BN,
                              seg_len=S, structure="uniform", seed=3)
    rng = np.random.default_rng(0)
    # every query row is the same vector, so all rows of a tile share one key order
    qrow = rng.standard_normal(d).astype(np.float32)
    k = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    q = np.tile(qrow, (1, 1, N, 1)).astype(np.float32)
    return w, {"q": q, "k": k, "v": k}, qrow


def _run(order_fn, n_chunks, lists="tile"):
    w, x, qrow = _problem()
    T = w.N // w.tile_m
    t = T - 1
    a = (t * w.tile_m // w.seg_len) * w.seg_len
    true_order = np.argsort(-(x["k"][0, 0, :a] @ qrow), kind="stable").astype(np.int32)
    ent = order_fn(true_order, a, w.tile_n)
    idx = np.zeros(1 << 12, np.int32)
    idx[:len(ent)] = ent
    exec_tiles = np.zeros((1, 1, T), np.int32)
    exec_tiles[0, 0, t] = ((t + 1) * w.tile_m - a) // w.tile_n + n_chunks
    return bench.ranking_study(w, x, lists, idx, lambda b, h, tt: 0, exec_tiles, [(0, 0, t)])


def test_true_order_scores_one():
    r = _run(lambda o, a, bn: o, n_chunks=2)
    assert r["tiles"] == 1
    assert r["overlap"] == 1.0 and r["mass"] == 1.0 and r["spearman"] == 1.0
    assert 0.0 < r["coverage"] < 1.0


def test_reversed_order():
    r = _run(lambda o, a, bn: o[::-1].copy(), n_chunks=1)
    assert r["overlap"] == 0.0 and r["mass"] < 0.25 and r["spearman"] == -1.0


def test_all_chunks_cover_everything():
    r = _run(lambda o, a, bn: o[::-1].copy(), n_chunks=256 // 64)
    assert r["coverage"] == 1.0 and r["overlap"] == 1.0 and r["mass"] == 1.0


def test_block_entries_expand_to_their_keys():
    # blocks in ascending order with every chunk executed: the whole history is covered
    r = _run(lambda o, a, bn: np.arange(a // bn, dtype=np.int32), n_chunks=256 // 64, lists="tile_blocks")
    assert r["coverage"] == 1.0 and r["overlap"] == 1.0


def test_refine_tau_brackets_the_budget():
    # a monotone MSE curve: mse(tau) = tau**2, budget 1e-6 -> boundary at 1e-3
    curve = lambda t: {"tau": t, "mse": t * t}
    sweep = [curve(t) for t in (1e-2, 2e-3, 5e-4, 0.0)]
    tau = bench.refine_tau(sweep, curve, budget=1e-6, steps=6)
    assert 5e-4 < tau <= 1e-3
    assert tau > 1e-3 * (2e-3 / 5e-4) ** (-1.0 / 64) * 0.999  # within one final bisection step
    assert all(r["mse"] <= 1e-6 for r in sweep if r.get("refined") and r["tau"] == tau)
    assert sum(1 for r in sweep if r.get("refined")) == 6


def test_refine_tau_without_bracket():
    curve = lambda t: {"tau": t, "mse": t * t}
    sweep = [curve(t) for t in (1e-4, 0.0)]  # every value within budget: nothing to refine
    assert bench.refine_tau(sweep, curve, budget=1e-6) == 1e-4
    sweep = [curve(t) for t in (1e-2, 5e-3)]  # none within budget
    assert bench.refine_tau(sweep, curve, budget=1e-6) is None


def test_stop_fired_share_counts_tiles_short_of_their_list():
    N, BM, BN, S = 1024, 128, 64, 256  # tiles 0,1 have no history; tile t has 2 + a_t/64 tiles in full
    T = N // BM
    t = np.arange(T)
    a = (t * BM // S) * S
    full = ((t + 1) * BM - a) // BN + a // BN
    ex = np.tile(full, (1, 2, 1)).astype(np.int32)   # [B=1, H=2, T]
    assert bench.stop_fired_share(ex, N, BM, BN, S) == 0.0
    ex[0, 1, 5] -= 1                                   # one of 12 tiles with history stops early
    assert abs(bench.stop_fired_share(ex, N, BM, BN, S) - 1 / 12) < 1e-12
    ex[0, 0, 0] = 1                                    # tiles without history never count
    assert abs(bench.stop_fired_share(ex, N, BM, BN, S) - 1 / 12) < 1e-12


def test_gather_figure_matches_committed_profile():
    """The gather bandwidth is the committed profile's bytes over the given time,
    and absent when the profile does not match the kernel source."""
    t = bench.traffic_figure()
    g = bench.gather_figure(100.0)
    if t is None:
        assert g is None
        return
    assert g["unit"] == "GB/s" and g["peak"] == bench.HBM_PEAK_GBS
    assert abs(g["achieved"] - t / 0.1 / 1e9) < 0.1
    assert abs(g["frac"] - g["achieved"] / bench.HBM_PEAK_GBS) < 1e-3


def test_mfma_busy_counter_reads_the_matching_profile():
    """The counter-based matrix-core share comes from the committed profile only
    when that profile was taken on the current attention source."""
    import json
    v = bench.mfma_busy_counter()
    try:
        rec = json.load(open(bench.COUNTERS_FILE))
    except OSError:
        assert v is None
        return
    if rec.get("kernel_source_sha256_16") != bench.source_hash(bench.ATTN_SOURCE):
        assert v is None
    else:
        assert v == round(rec["kernels"]["s2o_attn_fwd (S2O schedule)"]["mfma_busy"], 4)
        assert 0.0 < v < 1.0


def _run_by_tau(order_fn, chunks_by_tau):
    w, x, qrow = _problem()
    T = w.N // w.tile_m
    t = T - 1
    a = (t * w.tile_m // w.seg_len) * w.seg_len
    true_order = np.argsort(-(x["k"][0, 0, :a] @ qrow), kind="stable").astype(np.int32)
    idx = np.zeros(1 << 12, np.int32)
    idx[:a] = order_fn(true_order)
    p1 = ((t + 1) * w.tile_m - a) // w.tile_n
    exec_tiles = np.zeros((1, 1, T), np.int32)
    exec_tiles[0, 0, t] = p1 + max(chunks_by_tau.values())
    by_tau = {tau: [p1 + n] for tau, n in chunks_by_tau.items()}
    return bench.ranking_study(w, x, "tile", idx, lambda b, h, tt: 0, exec_tiles, [(0, 0, t)],
                               exec_by_tau=by_tau), a, w.tile_n


def test_by_tau_precision_and_recall_follow_the_definitions():
    # true order: the first chunk lies inside every row's important set (precision 1),
    # executing every chunk recalls all of it and covers the whole history
    r, a, bn = _run_by_tau(lambda o: o, {1e-2: 1, 0.0: 256 // 64})  # history 256 keys = 4 chunks
    rows = {e["tau"]: e for e in r["by_tau"]}
    assert [e["tau"] for e in r["by_tau"]] == [1e-2, 0.0]
    assert rows[1e-2]["precision"] == 1.0 and 0.0 < rows[1e-2]["recall"] < 1.0
    assert rows[0.0]["recall"] == 1.0 and rows[0.0]["coverage"] == 1.0
    assert rows[0.0]["precision"] < 1.0
    assert rows[1e-2]["coverage"] < rows[0.0]["coverage"]
    # reversed order: the first chunk holds the least important keys
    rr, _, _ = _run_by_tau(lambda o: o[::-1].copy(), {1e-2: 1})
    assert rr["by_tau"][0]["precision"] < rows[1e-2]["precision"]
    assert rr["by_tau"][0]["recall"] < rows[1e-2]["recall"]


def test_study_without_taus_has_no_table():
    r = _run(lambda o, a, bn: o, n_chunks=2)
    assert "by_tau" not in r


def test_amd_smi_sample_parses_clocks_and_power(monkeypatch):
    import json
    import subprocess
    out = {"gpu_data": [{"gpu": 0, "power": {"socket_power": {"value": 900, "unit": "W"}},
                         "clock": {**{f"gfx_{i}": {"clk": {"value": 1600 + 10 * i, "unit": "MHz"}} for i in range(8)},
                                   "mem_0": {"clk": {"value": 1900, "unit": "MHz"}}}}]}

    class R:
        stdout = json.dumps(out)
    monkeypatch.setattr(subprocess, "run", lambda *a, **k: R())
    clk, pw = bench.amd_smi_sample()
    assert clk == 1635.0 and pw == 900.0  # mean of the gfx clocks only


def test_clocks_under_load_summarises_samples(monkeypatch):
    readings = iter([(1600.0, 800.0), (1700.0, 1000.0)])
    monkeypatch.setattr(bench, "amd_smi_sample", lambda: next(readings, None))
    import torch
    monkeypatch.setattr(torch.cuda, "synchronize", lambda: None)
    monkeypatch.delenv("LD_PRELOAD", raising=False)
    r = bench.clocks_under_load(lambda: None, seconds=0.2)
    assert r["samples"] == 2 and r["gfx_mhz_mean"] == 1650 and r["gfx_mhz_min"] == 1600
    assert r["socket_power_w_mean"] == 900 and r["socket_power_w_max"] == 1000
    monkeypatch.setenv("LD_PRELOAD", "/opt/rocm/lib/librocprofiler-sdk-tool.so")
    assert bench.clocks_under_load(lambda: None, seconds=0.2) is None
