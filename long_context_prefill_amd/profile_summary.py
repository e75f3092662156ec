"""Summarise rocprofv3 CSV output into the short text kept under profiles/.

Usage: python -m long_context_prefill_amd.profile_summary KERNEL_STATS_CSV
           [--fetch COUNTER_CSV --write COUNTER_CSV --copy-bytes N] --command "..."
       python -m long_context_prefill_amd.profile_summary --counters CSV [CSV ...] --command "..."
Counter values (FETCH_SIZE, WRITE_SIZE, in KiB per dispatch) are scaled by what
the same counter reads for the plain copy kernel of known size in the same run.
--counters averages SQ counters per dispatch for the attention kernels and
derives matrix-core and wave-state shares from them (see counter_report).
"""

from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import sys


KERNELS = {  # kernel name -> the entry point that launches it
    "attn_kernel": None, "score_mfma_kernel": "s2o_score", "pool_kernel": "s2o_score",
    "segpool_kernel": "s2o_score", "pool_blocks_kernel": "s2o_score", "guide_kernel": "s2o_score",
    "query_score_kernel": "s2o_score", "minmax_kernel": "s2o_build_index",
    "hist_kernel": "s2o_build_index", "scan_kernel": "s2o_build_index",
    "scatter_kernel": "s2o_build_index", "range_sort_kernel": "s2o_build_index",
    "list_sort_kernel": "s2o_build_index", "queued_range_kernel": "s2o_build_index",
    "overflow_kernel": "s2o_build_index", "plan_kernel": "s2o_build_index",
    "query_sort_kernel": "s2o_build_index", "rocclr_copyBuffer": None,
}


def short(name: str) -> str:
    # the longest key wins: several kernel names contain a shorter one
    hits = [k for k in KERNELS if k in name]
    if not hits:
        return name[:60]
    key = max(hits, key=len)
    tail = name.split(key, 1)[1]
    if key == "attn_kernel":
        s2o = "ELb1E" in tail or ", true>" in tail
        return "s2o_attn_fwd (S2O schedule)" if s2o else "dense_attn_fwd"
    label = key + tail.split("(")[0] if key in ("hist_kernel", "scatter_kernel", "range_sort_kernel") else key
    return f"{label} ({KERNELS[key]})" if KERNELS[key] else key


def sources_hash(paths):
    """First 16 hex digits of the SHA-256 of the files' contents, concatenated in order."""
    h = hashlib.sha256()
    for path in paths:
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def per_kernel(path, value="Counter_Value"):
    agg = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        agg[r["Kernel_Name"]].append(float(r[value]))
    return agg


# MI355X: 256 CUs x 4 SIMDs in 32 shader engines.  SQ_BUSY_CYCLES sums the
# busy cycles of every shader engine; SQ_VALU_MFMA_BUSY_CYCLES and
# SQ_VALU_MFMA_COEXEC_CYCLES sum SIMD cycles; the SQ_WAVE_CYCLES / SQ_WAIT_* /
# SQ_ACTIVE_INST_ANY family sums wave cycles (in the same unit, so only their
# ratios are used).
SIMDS, SHADER_ENGINES = 1024, 32


def counter_report(paths):
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in paths:
        for r in csv.DictReader(open(path)):
            n = short(r["Kernel_Name"])
            if n in ("s2o_attn_fwd (S2O schedule)", "dense_attn_fwd"):
                per[n][r["Counter_Name"]].append(float(r["Counter_Value"]))
    out = {}
    for n, cs in per.items():
        avg = {c: sum(v) / len(v) for c, v in cs.items()}
        simd_cycles = avg["SQ_BUSY_CYCLES"] / SHADER_ENGINES * SIMDS
        wave = avg["SQ_WAVE_CYCLES"]
        out[n] = {
            "counters": avg,
            "mfma_busy": avg["SQ_VALU_MFMA_BUSY_CYCLES"] / simd_cycles,
            "mfma_valu_coexec": avg["SQ_VALU_MFMA_COEXEC_CYCLES"] / simd_cycles,
            "wave_issuing": avg["SQ_ACTIVE_INST_ANY"] / wave,
            "wave_waiting_issue": avg["SQ_WAIT_INST_ANY"] / wave,
            "wave_waiting_counters_barrier": avg["SQ_WAIT_ANY"] / wave,
            "valu_insts_per_mfma": (avg["SQ_INSTS_VALU"] - avg["SQ_INSTS_MFMA"]) / avg["SQ_INSTS_MFMA"],
            "trans_per_mfma": avg["SQ_INSTS_VALU_TRANS_F32"] / avg["SQ_INSTS_MFMA"],
            "lds_insts_per_mfma": avg["SQ_INSTS_LDS"] / avg["SQ_INSTS_MFMA"],
        }
        out[n].update(mfma_work(avg))
    return out


# SQ_INSTS_VALU_MFMA_MOPS_* count matrix-core operations in units of 512
# (one multiply-add is 2 flop).
MOPS_UNIT = 512


def mfma_work(avg):
    """Matrix-core flops by type and GPU-active cycles, when collected."""
    d = {}
    for t in ("BF16", "F32"):
        c = f"SQ_INSTS_VALU_MFMA_MOPS_{t}"
        if c in avg:
            d[f"mfma_flop_{t.lower()}"] = avg[c] * MOPS_UNIT
    if "GRBM_GUI_ACTIVE" in avg:
        d["gui_active_cycles"] = avg["GRBM_GUI_ACTIVE"]
    return d


def print_mfma_work(d):
    for t in ("bf16", "f32"):
        if f"mfma_flop_{t}" in d:
            print(f"  matrix-core work ({t})           {d[f'mfma_flop_{t}']:10.4g} flop "
                  f"(SQ_INSTS_VALU_MFMA_MOPS_{t.upper()} x {MOPS_UNIT})")
    if "gui_active_cycles" in d:
        print(f"  GPU active cycles                {d['gui_active_cycles']:10.4g} (GRBM_GUI_ACTIVE)")


# MI355X has 256 CUs; a wave64 vector instruction holds its SIMD for 4 cycles
# at full rate (transcendentals take longer, so the busy share below is a floor).
CUS = 256


def kernel_counter_table(paths, kernels):
    """Per-dispatch SQ counter averages of the named kernels (short names) and
    the shares derived from them: vector unit busy (SQ_INSTS_VALU x 4 cycles
    over SIMD cycles), LDS busy (SQ_LDS_IDX_ACTIVE per CU over SE busy
    cycles), bank-conflict share of LDS-active cycles, and the wave-time
    split.  A share is left out when its counters were not collected."""
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in paths:
        for r in csv.DictReader(open(path)):
            n = short(r["Kernel_Name"])
            if n in kernels:
                per[n][r["Counter_Name"]].append(float(r["Counter_Value"]))
    out = {}
    for n in kernels:
        if n not in per:
            continue
        avg = {c: sum(v) / len(v) for c, v in per[n].items()}
        d = {"counters": avg}
        if "SQ_BUSY_CYCLES" in avg:
            se = avg["SQ_BUSY_CYCLES"] / SHADER_ENGINES
            if "SQ_INSTS_VALU" in avg:
                d["valu_busy"] = avg["SQ_INSTS_VALU"] * 4 / (se * SIMDS)
            if "SQ_LDS_IDX_ACTIVE" in avg:
                d["lds_busy"] = avg["SQ_LDS_IDX_ACTIVE"] / CUS / se
        if "SQ_LDS_IDX_ACTIVE" in avg and "SQ_LDS_BANK_CONFLICT" in avg and avg["SQ_LDS_IDX_ACTIVE"] > 0:
            d["lds_bank_conflict_share"] = avg["SQ_LDS_BANK_CONFLICT"] / avg["SQ_LDS_IDX_ACTIVE"]
        d.update(mfma_work(avg))
        if all(c in avg for c in ("SQ_WAVE_CYCLES", "SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY")):
            w = avg["SQ_WAVE_CYCLES"]
            d["wave_issuing"] = avg["SQ_ACTIVE_INST_ANY"] / w
            d["wave_waiting_issue"] = avg["SQ_WAIT_INST_ANY"] / w
            d["wave_waiting_counters_barrier"] = avg["SQ_WAIT_ANY"] / w
        out[n] = d
    return out


def l2_report(a, copy, avg):
    """Per kernel: L2 hit rate TCC_HIT / (TCC_HIT + TCC_MISS), and the bytes of
    requests L2 sends towards DRAM addresses: TCC_EA0_RDREQ_DRAM_32B counts
    32-byte read sectors and TCC_EA0_WRREQ_DRAM 64-byte write requests (for the
    plain copy kernel of a.copy_bytes both come to exactly that many bytes; the
    scale below checks it).  Counters are averaged over a kernel's dispatches,
    except the copy's, whose largest dispatch is the calibration copy.  Prints a
    table and returns {kernel: {...}}."""
    def counters(path):
        per = collections.defaultdict(lambda: collections.defaultdict(list))
        for r in csv.DictReader(open(path)):
            per[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
        return per

    def mean(v):
        return sum(v) / len(v)

    def copy_value(per, counter):
        return max(max(per[k][counter]) for k in per if "copyBuffer" in k)

    out = collections.defaultdict(dict)
    if a.hitmiss:
        for k, c in counters(a.hitmiss).items():
            hit, miss = mean(c.get("TCC_HIT_sum", [0.0])), mean(c.get("TCC_MISS_sum", [0.0]))
            if hit + miss > 0:
                out[short(k)]["l2_hit_rate"] = hit / (hit + miss)
    for path, counter, unit, key, what in ((a.dram_read, "TCC_EA0_RDREQ_DRAM_32B_sum", 32.0, "dram_read_bytes", "reads"),
                                           (a.dram_write, "TCC_EA0_WRREQ_DRAM_sum", 64.0, "dram_write_bytes", "writes")):
        if not path:
            continue
        per = counters(path)
        scale = a.copy_bytes / (unit * copy_value(per, counter))
        print(f"calibration: plain copy {what} {unit * copy_value(per, counter) / 1e9:.4f} GB of DRAM-destined "
              f"requests ({counter} x {unit:.0f} B) -> scale x{scale:.3f}")
        for k, c in per.items():
            if counter in c:
                out[short(k)][key] = unit * (max(c[counter]) if "copyBuffer" in k else mean(c[counter])) * scale
    print(f"\n{'kernel':44s} {'L2 hit':>7s} {'DRAM rd GB':>11s} {'DRAM wr GB':>11s} {'GB/s':>8s}")
    for n, r in out.items():
        if n.startswith("at::") or "void at" in n:
            continue
        ms = avg.get(n)
        rd, wr = r.get("dram_read_bytes"), r.get("dram_write_bytes")
        bw = (rd + wr) / (ms * 1e-3) / 1e9 if (ms and rd is not None and wr is not None) else float("nan")
        hit = r.get("l2_hit_rate")
        print(f"{n:44s} {100 * hit if hit is not None else float('nan'):6.1f}% "
              f"{rd / 1e9 if rd is not None else float('nan'):11.2f} "
              f"{wr / 1e9 if wr is not None else float('nan'):11.2f} {bw:8.0f}")
    return out


def main_kernel_counters(a):
    print(f"command: {a.command}\n")
    for n, d in kernel_counter_table(a.counters, a.kernels).items():
        print(f"{n}: per dispatch")
        for c, v in sorted(d["counters"].items()):
            print(f"  {c:32s} {v:14.4g}")
        if "valu_busy" in d:
            print(f"  vector unit busy (full-rate floor) {100 * d['valu_busy']:6.1f} % of SIMD cycles")
        if "lds_busy" in d:
            print(f"  LDS busy                           {100 * d['lds_busy']:6.1f} % of CU cycles")
        if "lds_bank_conflict_share" in d:
            print(f"  bank conflicts                     {100 * d['lds_bank_conflict_share']:6.1f} % of LDS-active cycles")
        print_mfma_work(d)
        if "wave_issuing" in d:
            print(f"  wave time issuing / waiting for an issue slot / at waits and barriers: "
                  f"{100 * d['wave_issuing']:.0f} / {100 * d['wave_waiting_issue']:.0f} / "
                  f"{100 * d['wave_waiting_counters_barrier']:.0f} %")
        print()


def main_counters(a):
    print(f"command: {a.command}\n")
    rep = counter_report(a.counters)
    for n, r in rep.items():
        print(f"{n}: per dispatch")
        for c, v in sorted(r["counters"].items()):
            print(f"  {c:32s} {v:14.4g}")
        print(f"  matrix cores busy                {100 * r['mfma_busy']:6.1f} % of SIMD cycles "
              f"(SQ_VALU_MFMA_BUSY_CYCLES / (SQ_BUSY_CYCLES / {SHADER_ENGINES} x {SIMDS}))")
        print(f"  vector and matrix co-issuing     {100 * r['mfma_valu_coexec']:6.1f} % of SIMD cycles")
        print(f"  wave time issuing / waiting for an issue slot / at waits and barriers: "
              f"{100 * r['wave_issuing']:.0f} / {100 * r['wave_waiting_issue']:.0f} / "
              f"{100 * r['wave_waiting_counters_barrier']:.0f} %")
        print(f"  per MFMA: {r['valu_insts_per_mfma']:.2f} other VALU ({r['trans_per_mfma']:.2f} "
              f"transcendental), {r['lds_insts_per_mfma']:.2f} LDS instructions")
        print_mfma_work(r)
        print()
    if a.json_out:
        src = sources_hash(a.source) if a.source else None
        out = {n: {k: v for k, v in r.items() if k != "counters"} for n, r in rep.items()}
        json.dump({"kernels": out, "command": a.command, "kernel_source_sha256_16": src},
                  open(a.json_out, "w"), indent=1)


def main():
    if "--counters" in sys.argv:
        ap = argparse.ArgumentParser()
        ap.add_argument("--counters", nargs="+", required=True)
        ap.add_argument("--command", required=True)
        ap.add_argument("--json-out", help="also write the derived shares as JSON")
        ap.add_argument("--source", nargs="+", help="kernel sources whose hash the JSON records")
        ap.add_argument("--kernels", nargs="+", help="short kernel names: a generic table for these")
        a = ap.parse_args()
        if a.kernels:
            main_kernel_counters(a)
        else:
            main_counters(a)
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("stats")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-bytes", type=float, default=float(1 << 30))
    ap.add_argument("--command", required=True)
    ap.add_argument("--json-out")
    ap.add_argument("--traffic-out", help="write the S2O attention kernel's traffic record (JSON) here")
    ap.add_argument("--workload", default="", help="workload named in the traffic record")
    ap.add_argument("--source", nargs="+", help="kernel sources whose hash the traffic record holds")
    ap.add_argument("--hitmiss", help="counter CSV with TCC_HIT_sum and TCC_MISS_sum")
    ap.add_argument("--dram-read", help="counter CSV with TCC_EA0_RDREQ_DRAM_sum and TCC_EA0_RDREQ_DRAM_32B_sum")
    ap.add_argument("--dram-write", help="counter CSV with TCC_EA0_WRREQ_DRAM_sum")
    a = ap.parse_args()
    print(f"command: {a.command}\n")
    print(f"{'kernel':44s} {'calls':>5s} {'avg ms':>10s} {'total ms':>10s} {'%':>6s}")
    rows = list(csv.DictReader(open(a.stats)))
    avg = {}
    for r in rows:
        n = short(r["Name"])
        avg[n] = float(r["AverageNs"]) / 1e6
        print(f"{n:44s} {r['Calls']:>5s} {float(r['AverageNs']) / 1e6:10.3f} "
              f"{float(r['TotalDurationNs']) / 1e6:10.2f} {float(r['Percentage']):6.2f}")
    if not (a.fetch and a.write):
        return
    f, w = per_kernel(a.fetch), per_kernel(a.write)
    copy = [k for k in f if "copyBuffer" in k][0]
    fscale = a.copy_bytes / max(f[copy]) / 1024  # bytes per KiB unit of FETCH_SIZE
    wscale = a.copy_bytes / max(w[copy]) / 1024
    print(f"\ncalibration: plain copy of {a.copy_bytes:.0f} B reads FETCH_SIZE {max(f[copy]):.0f} KiB,"
          f" WRITE_SIZE {max(w[copy]):.0f} KiB -> scale fetch x{fscale:.3f}, write x{wscale:.3f}")
    print(f"\n{'kernel':44s} {'fetch GB':>10s} {'write GB':>10s} {'avg ms':>8s} {'GB/s':>8s}")
    out = {}
    for k in f:
        n = short(k)
        fb = sum(f[k]) / len(f[k]) * 1024 * fscale
        wb = sum(w.get(k, [0])) / max(len(w.get(k, [0])), 1) * 1024 * wscale
        ms = avg.get(n)
        bw = (fb + wb) / (ms * 1e-3) / 1e9 if ms else float("nan")
        out[n] = {"fetch_bytes": fb, "write_bytes": wb, "avg_ms": ms}
        if n.startswith("at::") or "void at" in n:
            continue
        print(f"{n:44s} {fb / 1e9:10.2f} {wb / 1e9:10.2f} {ms if ms else float('nan'):8.3f} {bw:8.0f}")
    l2 = l2_report(a, copy, avg) if (a.hitmiss or a.dram_read or a.dram_write) else {}
    for n, r in l2.items():
        if n in out:
            out[n].update(r)
    if a.json_out:
        json.dump(out, open(a.json_out, "w"), indent=1)
    if a.traffic_out:
        k = out["s2o_attn_fwd (S2O schedule)"]
        rec = {"kernel": "s2o_attn_fwd (attn_kernel_bf16<d=128, 4 waves, S2O>)", "workload": a.workload,
               "fetch_bytes_per_launch": k["fetch_bytes"], "write_bytes_per_launch": k["write_bytes"],
               "hbm_bytes_per_launch": k["fetch_bytes"] + k["write_bytes"], "avg_ms": k["avg_ms"],
               "note": f"FETCH_SIZE x{fscale:.0f} and WRITE_SIZE x{wscale:.0f} (scales from a "
                       "plain copy in the same run); these count every request that leaves L2, "
                       "Infinity Cache hits included",
               "command": a.command, "kernel_source_sha256_16": sources_hash(a.source) if a.source else None}
        if "dram_read_bytes" in k and "dram_write_bytes" in k:
            rec["dram_bytes_per_launch"] = k["dram_read_bytes"] + k["dram_write_bytes"]
            rec["dram_note"] = ("TCC_EA0_RDREQ_DRAM_32B x 32 B + TCC_EA0_WRREQ_DRAM x 64 B (a plain copy "
                                "reads and writes exactly its size by them): requests that leave L2 for local "
                                "HBM addresses, Infinity Cache hits included (no counter here separates those "
                                "from HBM reads)")
        if "l2_hit_rate" in k:
            rec["l2_hit_rate"] = k["l2_hit_rate"]
        json.dump(rec, open(a.traffic_out, "w"), indent=1)
        open(a.traffic_out, "a").write("\n")


if __name__ == "__main__":
    main()
