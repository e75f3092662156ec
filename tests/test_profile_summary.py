"""CPU checks of the rocprofv3 summariser used for profiles/ (no GPU)."""

import csv

from long_context_prefill_amd import profile_summary as ps


def test_kernel_names_map_to_the_longest_key():
    ns = "void s2o::(anonymous namespace)::"
    assert ps.short(ns + "query_score_kernel<__bf16>(float const*)") == "query_score_kernel (s2o_score)"
    assert ps.short(ns + "score_mfma_kernel<__bf16, 128, 32, 2>(float const*)") == "score_mfma_kernel (s2o_score)"
    assert ps.short(ns + "segpool_kernel(float const*)") == "segpool_kernel (s2o_score)"
    assert ps.short(ns + "pool_kernel<float>(float const*)") == "pool_kernel (s2o_score)"
    assert ps.short(ns + "pool_blocks_kernel<float>(float const*)") == "pool_blocks_kernel (s2o_score)"
    assert ps.short(ns + "range_sort_kernel<2048>(int)") == "range_sort_kernel<2048> (s2o_build_index)"
    assert ps.short(ns + "queued_range_kernel(int)") == "queued_range_kernel (s2o_build_index)"
    assert ps.short(ns + "attn_kernel_bf16<128, 4, true>(x)") == "s2o_attn_fwd (S2O schedule)"
    assert ps.short(ns + "attn_kernel_bf16<128, 4, false>(x)") == "dense_attn_fwd"
    assert ps.short("some_other_kernel") == "some_other_kernel"


def test_kernel_counter_table_shares(tmp_path):
    """Shares follow from the counters: 32 shader engines of 1024 SIMDs and 256 CUs."""
    path = tmp_path / "c.csv"
    name = "void s2o::(anonymous namespace)::scatter_kernel<4096>(x)"
    rows = {"SQ_BUSY_CYCLES": 32 * 1000.0, "SQ_INSTS_VALU": 1024 * 1000.0 / 4 / 2,
            "SQ_LDS_IDX_ACTIVE": 256 * 250.0, "SQ_LDS_BANK_CONFLICT": 256 * 50.0,
            "SQ_WAVE_CYCLES": 100.0, "SQ_ACTIVE_INST_ANY": 40.0, "SQ_WAIT_INST_ANY": 35.0, "SQ_WAIT_ANY": 25.0}
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for c, v in rows.items():
            wr.writerow({"Kernel_Name": name, "Counter_Name": c, "Counter_Value": v})
    t = ps.kernel_counter_table([str(path)], ["scatter_kernel<4096> (s2o_build_index)"])
    d = t["scatter_kernel<4096> (s2o_build_index)"]
    assert abs(d["valu_busy"] - 0.5) < 1e-12
    assert abs(d["lds_busy"] - 0.25) < 1e-12
    assert abs(d["lds_bank_conflict_share"] - 0.2) < 1e-12
    assert (d["wave_issuing"], d["wave_waiting_issue"], d["wave_waiting_counters_barrier"]) == (0.4, 0.35, 0.25)


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for k, c, v in rows:
            wr.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_l2_report_scales_by_the_copy(tmp_path):
    """L2 hit rate is hits over hits plus misses; DRAM-destined bytes are 32-byte
    read sectors and 64-byte write requests, averaged over a kernel's dispatches
    except the copy's largest, which fixes the scale (here the copy's counters
    give exactly its size, so the scale is 1)."""
    import types
    attn = "void s2o::(anonymous namespace)::attn_kernel_bf16<128, 4, true>(x)"
    copy = "__amd_rocclr_copyBuffer"
    hm, rd, wr = tmp_path / "hm.csv", tmp_path / "rd.csv", tmp_path / "wr.csv"
    _counter_csv(hm, [(attn, "TCC_HIT_sum", 30.0), (attn, "TCC_MISS_sum", 70.0),
                      (attn, "TCC_HIT_sum", 50.0), (attn, "TCC_MISS_sum", 50.0)])
    # copy of 128 KiB: 4096 sectors of 32 B read, 2048 requests of 64 B written; a small copy beside it
    _counter_csv(rd, [(copy, "TCC_EA0_RDREQ_DRAM_32B_sum", 4096.0), (copy, "TCC_EA0_RDREQ_DRAM_32B_sum", 8.0),
                      (attn, "TCC_EA0_RDREQ_DRAM_32B_sum", 300.0), (attn, "TCC_EA0_RDREQ_DRAM_32B_sum", 100.0)])
    _counter_csv(wr, [(copy, "TCC_EA0_WRREQ_DRAM_sum", 2048.0), (copy, "TCC_EA0_WRREQ_DRAM_sum", 0.0),
                      (attn, "TCC_EA0_WRREQ_DRAM_sum", 16.0)])
    a = types.SimpleNamespace(hitmiss=str(hm), dram_read=str(rd), dram_write=str(wr), copy_bytes=128 * 1024.0)
    out = ps.l2_report(a, copy, {"s2o_attn_fwd (S2O schedule)": 1.0})
    r = out["s2o_attn_fwd (S2O schedule)"]
    assert abs(r["l2_hit_rate"] - 0.4) < 1e-12
    assert abs(r["dram_read_bytes"] - 32 * 200) < 1e-9
    assert abs(r["dram_write_bytes"] - 16 * 64) < 1e-9
    assert abs(out[ps.short(copy)]["dram_read_bytes"] - 128 * 1024) < 1e-9
    assert abs(out[ps.short(copy)]["dram_write_bytes"] - 128 * 1024) < 1e-9


def test_matrix_core_work_from_the_op_counters(tmp_path):
    """SQ_INSTS_VALU_MFMA_MOPS_* count operations in units of 512: a 32x32x16
    bf16 MFMA (32768 flop) is 64 of them, so 128 of them per executed tile give
    the tile's 4.19 MFLOP; GRBM_GUI_ACTIVE passes through."""
    path = tmp_path / "c.csv"
    attn = "void s2o::(anonymous namespace)::attn_kernel_bf16<128, 4, true>(x)"
    score = "void s2o::(anonymous namespace)::score_mfma_kernel<__bf16, 128, 32, 2>(x)"
    tiles = 1000
    _counter_csv(path, [(attn, "SQ_INSTS_VALU_MFMA_MOPS_BF16", tiles * 128 * 64.0),
                        (attn, "GRBM_GUI_ACTIVE", 5.0e6),
                        (score, "SQ_INSTS_VALU_MFMA_MOPS_F32", 8.0)])
    d = ps.mfma_work(ps.kernel_counter_table([str(path)], ["s2o_attn_fwd (S2O schedule)"])
                     ["s2o_attn_fwd (S2O schedule)"]["counters"])
    assert d["mfma_flop_bf16"] == tiles * 4 * 128 * 64 * 128 and d["gui_active_cycles"] == 5.0e6
    s = ps.kernel_counter_table([str(path)], ["score_mfma_kernel (s2o_score)"])["score_mfma_kernel (s2o_score)"]
    assert s["mfma_flop_f32"] == 8 * 512 and "mfma_flop_bf16" not in s
