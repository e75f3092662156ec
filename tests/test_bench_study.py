"""CPU checks of bench.py (no GPU): the ranking study's figures take their
extreme values on inputs whose true attention order is known, the tau
refinement and the stop-fired share follow their definitions, the profile
readers honour the source hash, and the stdout record of a full-size fake run
stays short enough for the driver to parse."""

import json

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


def _study(order_fn, chunks_by_tau, tau_star, blocks=False):
    """The study of one tile (the last) of the small problem, whose list is
    order_fn(true key order, history length, BN)."""
    w, x, qrow = _problem()
    T = w.N // w.tile_m
    t = T - 1
    tile = (0, 0, t)
    a = (t * w.tile_m // w.seg_len) * w.seg_len
    true_order = np.argsort(-(x["k"][0, 0, :a] @ qrow), kind="stable").astype(np.int32)
    p1 = ((t + 1) * w.tile_m - a) // w.tile_n
    form = {"lists": {tile: order_fn(true_order, a, w.tile_n)}, "blocks": blocks, "p1": {tile: p1},
            "exec": {tau: {tile: p1 + c} for tau, c in chunks_by_tau.items()}, "tau": tau_star, "rows": None}
    return bench.ranking_study(w, x, [(0, 0, 0), tile], {"f": form}, threads=2)["f"]


def test_true_order_scores_one():
    r = _study(lambda o, a, bn: o, {1e-3: 2}, 1e-3)
    assert r["tiles"] == 1  # the tile without history is skipped
    assert r["overlap"] == 1.0 and r["mass"] == 1.0 and r["spearman"] == 1.0
    assert 0.0 < r["coverage"] < 1.0


def test_reversed_order():
    r = _study(lambda o, a, bn: o[::-1].copy(), {1e-3: 1}, 1e-3)
    assert r["overlap"] == 0.0 and r["mass"] < 0.25 and r["spearman"] == -1.0


def test_all_chunks_cover_everything():
    r = _study(lambda o, a, bn: o[::-1].copy(), {0.0: 256 // 64}, 0.0)
    assert r["coverage"] == 1.0 and r["overlap"] == 1.0 and r["mass"] == 1.0


def test_block_entries_expand_to_their_keys():
    # blocks in ascending order with every chunk executed: the whole history is covered
    r = _study(lambda o, a, bn: np.arange(a // bn, dtype=np.int32), {0.0: 256 // 64}, 0.0, blocks=True)
    assert r["coverage"] == 1.0 and r["overlap"] == 1.0
    assert np.array_equal(bench.expand_entries(np.array([2, 0]), True, 4), [8, 9, 10, 11, 0, 1, 2, 3])


def test_by_tau_precision_and_recall_follow_the_definitions():
    # true order: the first chunk lies inside every row's important set (precision 1),
    # executing every chunk recalls all of it and covers the whole history
    r = _study(lambda o, a, bn: o, {1e-2: 1, 0.0: 256 // 64}, 1e-2)  # history 256 keys = 4 chunks
    rows = {e["tau"]: e for e in r["by_tau"]}
    assert [e["tau"] for e in r["by_tau"]] == [1e-2, 0.0]
    assert rows[1e-2]["precision"] == 1.0 and 0.0 < rows[1e-2]["recall"] < 1.0
    assert rows[0.0]["recall"] == 1.0 and rows[0.0]["coverage"] == 1.0
    assert rows[0.0]["precision"] < 1.0
    assert rows[1e-2]["coverage"] < rows[0.0]["coverage"]
    # reversed order: the first chunk holds the least important keys
    rr = _study(lambda o, a, bn: o[::-1].copy(), {1e-2: 1}, 1e-2)
    assert rr["by_tau"][0]["precision"] < rows[1e-2]["precision"]
    assert rr["by_tau"][0]["recall"] < rows[1e-2]["recall"]
    c = bench.compact_study({"tile": r})["tile"]  # at tau*, then bench.STUDY_TAUS = 1e-2, 3e-3, 1e-3
    assert c[0] == [round(rows[1e-2]["precision"], 3), round(rows[1e-2]["recall"], 3)]
    assert c[1] == c[0] and c[2] is None and c[3] is None


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


def test_sample_is_the_measurement_definition():
    w = synth.WORKLOADS["llama8b_n128k"]
    s = bench.sample_tiles(w)
    T, P = w.N // w.tile_m, w.seg_len // w.tile_m
    fixed = {(0, h, t) for h in (0, 9, 18, 27) for seg in range(T // P) for t in (seg * P, seg * P + P - 1)}
    assert fixed <= set(s) and len(fixed) == 4 * 2 * (T // P)
    assert 0 < len(set(s) - fixed) <= 16 and s == sorted(set(s))
    assert s == bench.sample_tiles(w)  # seeded


def test_gather_figure_matches_committed_profile():
    """The beyond-L2 bandwidth is the committed record's bytes over the given
    time, and absent when the record does not match the kernel source."""
    rec = bench.traffic_record()
    g = bench.gather_figure(100.0)
    if rec is None:
        assert g is None and bench.traffic_figure() is None
        return
    t = rec["hbm_bytes_per_launch"]
    assert abs(g["beyond_l2_gbs"] - t / 0.1 / 1e9) < 0.1
    assert abs(g["beyond_l2_frac"] - g["beyond_l2_gbs"] / bench.HBM_PEAK_GBS) < 1e-3
    if rec.get("dram_bytes_per_launch") is not None:
        assert abs(g["dram_gbs"] - rec["dram_bytes_per_launch"] / 0.1 / 1e9) < 0.1


def test_mfma_busy_counter_reads_the_matching_profile():
    """The counter-based matrix-core share comes from the committed profile only
    when that profile was taken on the current attention source."""
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


def test_amd_smi_sample_parses_clocks_and_power(monkeypatch):
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


# ----------------------------------------------------- the stdout record ------

def _fake_result(mode, rng, tau=1.4186124135047637e-3):
    sweep = [{"tau": float(t), "density": round(float(rng.random()), 4), "mse": float(rng.random() * 1e-4),
              "rel_mse": float(rng.random()), "max_abs_vs_dense": float(rng.random()),
              "stop_fired": float(rng.random())} for t in synth.TAU_SWEEP + (1.3e-3, 1.4e-3, 1.45e-3, 1.43e-3)]
    return {"mode": mode, "tau": tau, "ms_per_step": 107.0512345, "score_ms": 5.2512345, "sort_ms": 19.0612345,
            "attn_ms": 82.7412345, "step_stats": {"median": 107.051, "min": 106.912, "p90": 107.389},
            "executed": 19462857, "density": 0.5795123456, "mse": 9.8964123e-06, "rel_mse": 0.03212345678,
            "max_abs_vs_dense": 0.123456789, "stop_fired": 0.8123456789, "achieved": 1022.123456789,
            "sweep": sweep, "vs_dense": 1.1612345678,
            "at_rel_mse_budget": {"tau": 3e-4, "density": 0.9998, "rel_mse": 3.4e-6, "ms": 149.123456,
                                  "vs_dense": 0.8312345},
            "clocks": {"gfx_mhz_mean": 1655, "gfx_mhz_min": 1646, "gfx_mhz_max": 1672,
                       "socket_power_w_mean": 1368, "socket_power_w_max": 1390, "samples": 81,
                       "source": "amd-smi"}}


def test_record_of_a_full_run_fits_the_driver(monkeypatch):
    """Every field a default run produces, with full-precision floats: the
    stdout line stays under bench.RECORD_LIMIT characters and keeps the
    driver's fields, while the detail record holds the sweeps and the study."""
    monkeypatch.setattr(bench, "traffic_record", lambda: {
        "hbm_bytes_per_launch": 486483123456.789, "dram_bytes_per_launch": 123456789012.345,
        "l2_hit_rate": 0.612345678})
    rng = np.random.default_rng(5)
    w = synth.WORKLOADS["llama8b_n128k"]
    args = bench.parse(["--steps", "20", "--warmup", "5"])
    main = _fake_result("tile", rng)
    forms = {m: _fake_result(m, rng) for m in args.modes.split(",")}

    class Ctx:
        dense_ms = 124.6512345
    workloads = {"llama8b_n16k": bench.compact_workload(Ctx, [_fake_result("tile", rng, 5.6234567e-3)]),
                 "llama8b_n64k": bench.compact_workload(Ctx, [_fake_result("tile", rng, 1e-3)]),
                 "uniform_n128k": bench.compact_workload(Ctx, [_fake_result("tile", rng, 0.0),
                                                              _fake_result("tile", rng, 1e-3)])}
    parity = {"tiles": 144, "tau": main["tau"], "list_mismatch": 0, "exec_mismatch": 0, "near_tau": 1,
              "max_abs": 0.0123456789, "mean_abs": 0.000412345678, "ok": True, "dense_rows": 576,
              "dense_max_abs": 0.00812345678, "dense_mean_abs": 0.000312345678}
    cpu = {"value": 1384332.123, "unit": "ms", "cores": 16, "cpu": "AMD EPYC 9575F 64-Core Processor" + " " * 16,
           "kind": "oracle", "extrapolated": True,
           "sample": "144 tiles (heads 0,9,18,27 first+last tile of each segment, 16 seeded) at tau*: "
                     "12.34 s; scaled by executed keys 1245622848/5036224"}
    study = {}
    for m in ["tile"] + list(forms):
        by = [{"tau": r["tau"], "precision": float(rng.random()), "recall": float(rng.random()),
               "coverage": float(rng.random())} for r in main["sweep"]]
        study[m] = {"overlap": 0.7667, "mass": 0.8563, "coverage": 0.8047, "spearman": 0.3451, "tiles": 135,
                    "tau": main["tau"], "important_mass": 0.9, "by_tau": by}
    rec, full = bench.build_record(args, w, main, Ctx.dense_ms, forms, workloads, parity, cpu, study,
                                   70.1e9 * 7, 0.5967)
    line = json.dumps(rec, separators=(",", ":"))
    assert len(line) < bench.RECORD_LIMIT - 400, len(line)  # room for longer numbers or names
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline", "parity",
                "workloads", "forms", "ranking_study", "at_rel_mse_1e-5"):
        assert key in rec, key
    assert rec["roofline"]["frac"] == round(main["achieved"] / bench.BF16_MFMA_PEAK_TFLOPS, 4)
    assert set(rec["ranking_study"]["precision_recall"]) == {"tile", "segment", "blocks", "qperm", "shared"}
    assert "tau_sweep" in full and "form_sweeps" in full and "by_tau" in full["ranking_study"]["tile"]
    assert json.loads(line) == rec


def test_host_cpu_model_reads_the_first_model_name(tmp_path):
    f = tmp_path / "cpuinfo"
    f.write_text("processor\t: 0\nvendor_id\t: X\nmodel name\t: Some  CPU   @ 2.70GHz\n\n"
                 "processor\t: 1\nmodel name\t: Other\n")
    assert bench.host_cpu_model(str(f)) == "Some CPU @ 2.70GHz"
    f.write_text("processor\t: 0\n")
    assert bench.host_cpu_model(str(f)) is None
    assert bench.host_cpu_model(str(tmp_path / "missing")) is None
