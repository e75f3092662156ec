"""CPU checks of the parity comparison itself (tests/parity_util.compare): fed the
oracle's own results it reports nothing, and each planted mistake in the
"device" side (a swapped list entry, an early stop far from tau, a wrong output
value) is reported as exactly that kind of mismatch; a stop that floating point
decides within 1e-4 of tau is counted as near-tau and its output re-checked
against the oracle forced to the same chunk count."""

import numpy as np
import pytest
import torch

import oracle
from long_context_prefill_amd import synth
import parity_util as pu


class OracleRun:
    """Stands in for parity_util.GpuRun with the oracle's lists on the CPU."""

    def __init__(self, w, x, qperm=False):
        self.w, self.x = w, x
        self.po = oracle.problem_from_workload(w, qperm=qperm)
        self.lists = oracle.lists_all(self.po, oracle.scores_all(self.po, x["q"], x["k"]))

    def tile_list(self, b, h, t):
        off = oracle.list_offset(self.po, b, h, t)
        return self.lists[off:off + oracle.list_len(self.po, t)].copy()


def device_side(run, tiles, tau, force=None):
    """Outputs and executed-chunk counts as the HIP path returns them, taken from
    the oracle (optionally forced to a chunk count per tile)."""
    w, po = run.w, run.po
    T = w.N // w.tile_m
    res = oracle.attn_tiles(po, run.x["q"], run.x["k"], run.x["v"], tiles, tau, force_n=force)
    o = torch.zeros(w.B, w.Hq, w.N, w.d, dtype=torch.float32)
    ex = torch.zeros(w.B, w.Hq, T, dtype=torch.int32)
    for n, (b, h, t) in enumerate(tiles):
        rows = res["rows"][n] if res["rows"] is not None else np.arange(t * w.tile_m, (t + 1) * w.tile_m)
        o[b, h][torch.as_tensor(rows)] = torch.from_numpy(res["out"][n]).float()
        ex[b, h, t] = int(res["n_exec"][n])
    return o, ex


@pytest.fixture(scope="module")
def case(oracle_lib):
    w = synth.custom_workload(B=1, Hq=2, Hkv=1, N=512, d=64, dtype="f32", tile_m=64, tile_n=64,
                              seg_len=256, seed=31)
    x = synth.make_inputs(w)
    run = OracleRun(w, x)
    tiles = [(0, h, t) for h in range(w.Hq) for t in range(w.N // w.tile_m)]
    return w, x, run, tiles


TAU = 1e-3


def test_identical_results_report_nothing(case):
    w, x, run, tiles = case
    o, ex = device_side(run, tiles, TAU)
    rep = pu.compare(run, tiles, TAU, o, ex)
    assert (rep["list_mismatch"], rep["exec_mismatch"], rep["near_tau"]) == (0, 0, 0), rep
    assert rep["n"] == len(tiles) * w.tile_m * w.d
    assert rep["max_abs"] < 1e-6
    pu.assert_report(rep, "f32")


def test_identical_results_with_the_query_permutation(case):
    w, x, _, tiles = case
    run = OracleRun(w, x, qperm=True)
    o, ex = device_side(run, tiles, TAU)
    rep = pu.compare(run, tiles, TAU, o, ex)
    assert rep["max_abs"] < 1e-6 and rep["n"] == len(tiles) * w.tile_m * w.d, rep
    pu.assert_report(rep, "f32")
    # The same outputs read in plain row order do not match: the rows map matters.
    plain = OracleRun(w, x)
    rep2 = pu.compare(plain, tiles, TAU, o, ex, check_lists=False)
    assert rep2["max_abs"] > 1e-4 or rep2["exec_mismatch"] > 0


def test_a_swapped_list_entry_is_a_list_mismatch(case):
    w, x, run, tiles = case
    o, ex = device_side(run, tiles, TAU)
    t = w.N // w.tile_m - 1
    off = oracle.list_offset(run.po, 0, 1, t)
    bad = OracleRun.__new__(OracleRun)
    bad.__dict__.update(run.__dict__)
    bad.lists = run.lists.copy()
    bad.lists[off], bad.lists[off + 1] = bad.lists[off + 1], bad.lists[off]
    rep = pu.compare(bad, tiles, TAU, o, ex)
    assert rep["list_mismatch"] == 1 and rep["exec_mismatch"] == 0, rep
    with pytest.raises(AssertionError):
        pu.assert_report(rep, "f32")


def test_an_early_stop_far_from_tau_is_an_exec_mismatch(case):
    w, x, run, tiles = case
    res = oracle.attn_tiles(run.po, x["q"], x["k"], x["v"], tiles, TAU)
    n = int(np.argmax(res["chunks"]))
    assert res["chunks"][n] >= 2
    g = res["gstar"][n, res["chunks"][n] - 2]
    assert abs(g - TAU) > 1e-3 * TAU      # the gain there is not a floating-point call
    o, ex = device_side(run, tiles, TAU)
    b, h, t = tiles[n]
    ex[b, h, t] -= 1
    rep = pu.compare(run, tiles, TAU, o, ex)
    assert rep["exec_mismatch"] == 1 and rep["near_tau"] == 0, rep
    with pytest.raises(AssertionError):
        pu.assert_report(rep, "f32")


def test_a_stop_within_the_near_tau_band_is_rechecked_at_the_gpu_count(case):
    w, x, run, tiles = case
    res0 = oracle.attn_tiles(run.po, x["q"], x["k"], x["v"], tiles, TAU)
    n = int(np.argmax(res0["chunks"]))
    g0 = float(res0["gstar"][n, 0])
    # tau just under the first chunk's gain: the oracle goes on, a device whose
    # rounding put the gain under tau stops after one chunk.
    tau = g0 * (1 - 0.5 * pu.NEAR_TAU_REL)
    res = oracle.attn_tiles(run.po, x["q"], x["k"], x["v"], tiles, tau)
    assert res["chunks"][n] >= 2
    p1 = int(res["n_exec"][n]) - int(res["chunks"][n])
    force = [0] * len(tiles)
    force[n] = 1
    o, ex = device_side(run, tiles, tau, force=force)
    b, h, t = tiles[n]
    assert int(ex[b, h, t]) == p1 + 1
    rep = pu.compare(run, tiles, tau, o, ex)
    assert rep["near_tau"] == 1 and rep["exec_mismatch"] == 0, rep
    assert rep["max_abs"] < 1e-6, rep
    pu.assert_report(rep, "f32")
    # The stopped tile's output is re-checked: a wrong value there is caught.
    o[b, h, t * w.tile_m + 3, 5] += 1e-3
    rep = pu.compare(run, tiles, tau, o, ex)
    assert rep["near_tau"] == 1 and rep["max_abs"] > 1e-4, rep
    with pytest.raises(AssertionError):
        pu.assert_report(rep, "f32")


def test_a_wrong_output_value_exceeds_the_tolerance(case):
    w, x, run, tiles = case
    o, ex = device_side(run, tiles, TAU)
    o[0, 0, 100, 7] += 2e-4
    rep = pu.compare(run, tiles, TAU, o, ex)
    assert rep["list_mismatch"] == 0 and rep["exec_mismatch"] == 0
    assert abs(rep["max_abs"] - 2e-4) < 1e-6, rep
    with pytest.raises(AssertionError):
        pu.assert_report(rep, "f32")


def test_bf16_tolerance_checks_the_mean_as_well():
    n = 1000
    ok = dict(list_mismatch=0, exec_mismatch=0, max_abs=1e-2, sum_abs=1.0, n=n, mean_abs=1e-3)
    pu.assert_report(ok, "bf16")
    with pytest.raises(AssertionError):
        pu.assert_report(dict(ok, mean_abs=3e-3), "bf16")
    with pytest.raises(AssertionError):
        pu.assert_report(dict(ok, max_abs=3e-2), "bf16")
