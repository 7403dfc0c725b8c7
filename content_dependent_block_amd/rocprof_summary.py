"""Summaries of rocprofv3 CSV output for the kernels of this library.

    python -m content_dependent_block_amd.rocprof_summary stats <trace_dir>
    python -m content_dependent_block_amd.rocprof_summary traffic \\
        --fetch <dir> --write <dir> --copy-fetch <dir> --copy-write <dir> \\
        --kernel <regex> --stage <name> --workload <name> \\
        [--json <out.json>]

`stats` prints the per-kernel table of a `--kernel-trace --stats` run.
`traffic` turns FETCH_SIZE / WRITE_SIZE (KiB per dispatch) into HBM bytes per
launch of one kernel.  Each counter is scaled by what the same counter reads
for a plain device copy of known size (bench.py --copy-calibration: 1 GiB read,
1 GiB written per launch), so the figure is in bytes whatever the counter's
sampling scope.  With --json it writes the record bench.py reads for the
roofline's `traffic` field; the record carries the hash of the kernel's source
so a later change of the kernel invalidates it.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "content_dependent_block_amd", "csrc")

# stage name (bench.py) -> kernel source file
STAGE_SOURCES = {
    "block_pool": "block_pool.hip",
    "coarse_score": "coarse_score.hip",
    "topk_select": "topk_select.hip",
    "coarse_select": "coarse_score.hip",
    "sparse_flash_fwd": "fine_gather.hip",
    "gather_index": "fine_gather.hip",
    "gather_combine": "fine_gather.hip",
    "bwd_prep": "fine_backward.hip",
    "bwd_index": "fine_gather.hip",
    "bwd_pairs": "fine_backward.hip",
    "bwd_reduce": "fine_backward.hip",
}

_SHORT = re.compile(r"(gather_partial_kernel|combine_kernel|topk_lane_kernel|topk_wave_kernel|"
                    r"coarse_select_kernel|coarse_panel_kernel|bucket_count_kernel|bucket_scan_kernel|"
                    r"bucket_fill_kernel|block_pool_kernel|zero_i32_kernel|sparse_flash_kernel|"
                    r"elementwise_kernel|bwd_prep_kernel|bwd_pair_kernel|bwd_dq_kernel|bwd_dkv_kernel)")


def short(name: str) -> str:
    m = _SHORT.search(name)
    return m.group(1) if m else name[:48]


def source_sha(stage: str) -> str:
    with open(os.path.join(CSRC, STAGE_SOURCES[stage]), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _one(d: str, pattern: str) -> str:
    hits = glob.glob(os.path.join(d, "**", pattern), recursive=True)
    if not hits:
        raise SystemExit(f"no {pattern} under {d}")
    return hits[0]


def stats(d: str):
    rows = []
    for r in csv.DictReader(open(_one(d, "*kernel_stats.csv"))):
        rows.append((short(r["Name"]), int(r["Calls"]), float(r["TotalDurationNs"]) / 1e3,
                     float(r["AverageNs"]) / 1e3, float(r["Percentage"])))
    return rows


def counter_per_dispatch(d: str, counter: str, kernel_re: str):
    """Mean over matching dispatches of the counter (summed over its instances)."""
    per = collections.defaultdict(float)
    for r in csv.DictReader(open(_one(d, "*counter_collection.csv"))):
        if r["Counter_Name"] != counter or not re.search(kernel_re, r["Kernel_Name"]):
            continue
        per[r["Dispatch_Id"]] += float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} records for /{kernel_re}/ under {d}")
    return sum(per.values()) / len(per), len(per)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    t = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        t.add_argument("--" + k.replace("_", "-"), required=True)
    t.add_argument("--kernel", required=True, help="regex on the kernel name")
    t.add_argument("--stage", required=True, choices=sorted(STAGE_SOURCES))
    t.add_argument("--workload", required=True)
    t.add_argument("--copy-bytes", type=float, default=float(1 << 30))
    t.add_argument("--json")
    a = ap.parse_args(argv)

    if a.cmd == "stats":
        print(f"{'kernel':34s} {'calls':>6s} {'total_us':>11s} {'avg_us':>10s} {'pct':>7s}")
        for n, c, tot, avg, pct in stats(a.dir):
            print(f"{n:34s} {c:6d} {tot:11.1f} {avg:10.2f} {pct:7.2f}")
        return 0

    copy_re = r"elementwise|copy|mul"
    cf, _ = counter_per_dispatch(a.copy_fetch, "FETCH_SIZE", copy_re)
    cw, _ = counter_per_dispatch(a.copy_write, "WRITE_SIZE", copy_re)
    kf, nf = counter_per_dispatch(a.fetch, "FETCH_SIZE", a.kernel)
    kw, nw = counter_per_dispatch(a.write, "WRITE_SIZE", a.kernel)
    f_scale = a.copy_bytes / cf     # bytes per counter unit, reads
    w_scale = a.copy_bytes / cw     # bytes per counter unit, writes
    rec = {
        "stage": a.stage, "kernel_regex": a.kernel, "workload": a.workload,
        "source_sha": source_sha(a.stage),
        "fetch_counter_per_launch": kf, "write_counter_per_launch": kw,
        "copy_fetch_counter": cf, "copy_write_counter": cw,
        "fetch_bytes_per_unit": f_scale, "write_bytes_per_unit": w_scale,
        "fetch_bytes_per_launch": kf * f_scale, "write_bytes_per_launch": kw * w_scale,
        "hbm_bytes_per_launch": kf * f_scale + kw * w_scale,
        "dispatches": [nf, nw],
    }
    print(json.dumps(rec, indent=1))
    if a.json:
        with open(a.json, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
