"""Summarise rocprofv3 CSV output into the short text kept under profiles/.

Usage: python -m long_context_prefill_amd.profile_summary KERNEL_STATS_CSV
           [--fetch COUNTER_CSV --write COUNTER_CSV --copy-bytes N] --command "..."
Counter values (FETCH_SIZE, WRITE_SIZE, in KiB per dispatch) are scaled by what
the same counter reads for the plain copy kernel of known size in the same run.
"""

from __future__ import annotations

import argparse
import collections
import csv
import json


def short(name: str) -> str:
    for key in ("attn_kernel", "score_kernel", "pool_blocks_kernel", "pool_kernel", "minmax_kernel",
                "hist_kernel", "scan_kernel", "scatter_kernel", "range_sort_kernel", "list_sort_kernel",
                "overflow_kernel", "plan_kernel", "rocclr_copyBuffer"):
        if key in name:
            tail = name.split(key, 1)[1]
            if key == "attn_kernel":
                s2o = "ELb1E" in tail or ", true>" in tail
                return "s2o_attn_fwd (S2O schedule)" if s2o else "dense_attn_fwd"
            if key in ("hist_kernel", "scatter_kernel", "range_sort_kernel"):
                return key + tail.split("(")[0] + " (s2o_build_index)"
            if key in ("minmax_kernel", "scan_kernel", "list_sort_kernel", "overflow_kernel", "plan_kernel"):
                return key + " (s2o_build_index)"
            if key == "score_kernel":
                return "score_kernel (s2o_score)"
            if key == "pool_kernel":
                return "pool_kernel (s2o_score)"
            return key
    return name[:60]


def per_kernel(path, value="Counter_Value"):
    agg = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        agg[r["Kernel_Name"]].append(float(r[value]))
    return agg


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("stats")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-bytes", type=float, default=float(1 << 30))
    ap.add_argument("--command", required=True)
    ap.add_argument("--json-out")
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
    if a.json_out:
        json.dump(out, open(a.json_out, "w"), indent=1)


if __name__ == "__main__":
    main()
