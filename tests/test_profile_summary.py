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
