"""Summaries of rocprofv3 CSV output for the kernels of this library.

    python -m content_dependent_block_amd.rocprof_summary stats <trace_dir>
    python -m content_dependent_block_amd.rocprof_summary traffic \\
        --read <dir> --write <dir> --copy-read <dir> --copy-write <dir> \\
        --kernel <regex> --stage <name> --workload <name> [--json <out.json>]
    python -m content_dependent_block_amd.rocprof_summary counters <dir> [<dir> ...] \\
        --kernel <regex> [--kernel <regex> ...]

`stats` prints the per-kernel table of a `--kernel-trace --stats` run.

`traffic` gives the HBM-side bytes per launch of one kernel from the L2's
requests to the memory fabric, one --pmc pass each:
    read bytes  = 32 TCC_EA0_RDREQ_32B_sum + 64 TCC_EA0_RDREQ_64B_sum
                  + 128 TCC_EA0_RDREQ_128B_sum
    write bytes = 1024 WRITE_SIZE (KiB)
(The stock FETCH_SIZE takes its 128-byte term from TCC_BUBBLE, which counts
nothing on gfx950, and so counts a 128-byte request as 64 bytes.)  The same
passes over a plain device copy of 1 GiB (bench.py --copy-calibration; its
dispatches that read under half of that, the buffer fills, are left out) check
the formulas: the record carries counted / true bytes of the copy, 1.0 when
they hold, and is not scaled by it.  With --json it writes the record bench.py
reads for the roofline's `traffic` field; the record carries the hash of the
kernel's source so a later change of the kernel invalidates it.

`counters` averages SQ and GRBM counters per dispatch of each kernel over the
given --pmc passes and derives, with C = GRBM_GUI_ACTIVE / 8 (the counter is
summed over the 8 XCDs) the kernel's cycles and 1024 SIMDs:
    VALU, SALU, LDS, MFMA instructions per wave  = SQ_INSTS_* / SQ_WAVES
    MFMA busy  = SQ_VALU_MFMA_BUSY_CYCLES / (C * 1024)
    VALU busy  = 4 SQ_ACTIVE_INST_VALU / (C * 1024)
    LDS busy   = 4 SQ_ACTIVE_INST_LDS / (C * 1024)
    bf16 MFMA FLOP = 512 SQ_INSTS_VALU_MFMA_MOPS_BF16
    LDS bank-conflict cycles per LDS instruction = SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS
    L2 hit rate = TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum)
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
    "static_combine": "sparse_flash_fwd.hip",
    "bwd_prep": "fine_backward.hip",
    "bwd_index": "fine_gather.hip",
    "bwd_pairs": "fine_backward.hip",
    "bwd_reduce": "fine_backward.hip",
}

_SHORT = re.compile(r"(gather_partial_kernel|static_item_kernel|static_combine_kernel|combine_kernel|"
                    r"topk_lane_kernel|topk_wave_kernel|coarse_select_kernel|coarse_repair_kernel|coarse_panel_kernel|"
                    r"bucket_count_kernel|bucket_scan_small_kernel|bucket_scan_kernel|bucket_fill_kernel|block_pool_kernel|"
                    r"zero_i32_kernel|sparse_flash_kernel|per_query_kernel|pad_rows_kernel|unpad_rows_kernel|"
                    r"elementwise_kernel|reduce_kernel|bwd_prep_kernel|bwd_pair_kernel|bwd_dq_kernel|bwd_dkv_kernel|"
                    r"copyBuffer)")


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


def per_dispatch(d: str, kernel_re: str):
    """{dispatch id: {counter: value summed over its instances}} of the
    dispatches whose kernel name matches."""
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    for r in csv.DictReader(open(_one(d, "*counter_collection.csv"))):
        if re.search(kernel_re, r["Kernel_Name"]):
            per[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no counter records for /{kernel_re}/ under {d}")
    return per


def read_bytes(c) -> float:
    return (32 * c.get("TCC_EA0_RDREQ_32B_sum", 0.0) + 64 * c.get("TCC_EA0_RDREQ_64B_sum", 0.0)
            + 128 * c.get("TCC_EA0_RDREQ_128B_sum", 0.0))


def write_bytes(c) -> float:
    return 1024 * c.get("WRITE_SIZE", 0.0)


def mean(xs):
    xs = list(xs)
    return sum(xs) / len(xs) if xs else float("nan")


COPY_RE = r"elementwise|copy"


def traffic(a):
    cr = [read_bytes(c) for c in per_dispatch(a.copy_read, COPY_RE).values()]
    cw = [write_bytes(c) for c in per_dispatch(a.copy_write, COPY_RE).values()]
    copies_r = [x for x in cr if x > a.copy_bytes / 2]
    copies_w = [x for x in cw if x > a.copy_bytes / 2]
    kr = [read_bytes(c) for c in per_dispatch(a.read, a.kernel).values()]
    kw = [write_bytes(c) for c in per_dispatch(a.write, a.kernel).values()]
    rb, wb = mean(kr), mean(kw)
    return {
        "stage": a.stage, "kernel_regex": a.kernel, "workload": a.workload,
        "source_sha": source_sha(a.stage),
        "read_formula": "32 TCC_EA0_RDREQ_32B_sum + 64 TCC_EA0_RDREQ_64B_sum + 128 TCC_EA0_RDREQ_128B_sum",
        "write_formula": "1024 WRITE_SIZE",
        "copy_read_ratio": round(mean(copies_r) / a.copy_bytes, 4),
        "copy_write_ratio": round(mean(copies_w) / a.copy_bytes, 4),
        "copy_dispatches": [len(copies_r), len(copies_w)],
        "fetch_bytes_per_launch": rb, "write_bytes_per_launch": wb,
        "hbm_bytes_per_launch": rb + wb,
        "dispatches": [len(kr), len(kw)],
    }


def counters(dirs, kernel_re):
    """Counter means per dispatch over every pass, and the derived figures."""
    acc = collections.defaultdict(list)
    for d in dirs:
        for c in per_dispatch(d, kernel_re).values():
            for name, v in c.items():
                acc[name].append(v)
    c = {k: mean(v) for k, v in acc.items()}
    out = {"raw": c}
    waves = c.get("SQ_WAVES")
    cyc = c["GRBM_GUI_ACTIVE"] / 8 if "GRBM_GUI_ACTIVE" in c else None
    if waves:
        for name in ("VALU", "SALU", "LDS", "MFMA"):
            if f"SQ_INSTS_{name}" in c:
                out[f"{name.lower()}_insts_per_wave"] = c[f"SQ_INSTS_{name}"] / waves
    if cyc:
        out["cycles"] = cyc
        out["us_at_2.4GHz"] = cyc / 2400.0
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
            out["mfma_busy"] = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * 1024)
        if "SQ_ACTIVE_INST_VALU" in c:
            out["valu_busy"] = 4 * c["SQ_ACTIVE_INST_VALU"] / (cyc * 1024)
        if "SQ_ACTIVE_INST_LDS" in c:
            out["lds_busy"] = 4 * c["SQ_ACTIVE_INST_LDS"] / (cyc * 1024)
    if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in c:
        out["bf16_mfma_flop"] = 512 * c["SQ_INSTS_VALU_MFMA_MOPS_BF16"]
    if "SQ_LDS_BANK_CONFLICT" in c and c.get("SQ_INSTS_LDS"):
        out["lds_conflict_cycles_per_lds_inst"] = c["SQ_LDS_BANK_CONFLICT"] / c["SQ_INSTS_LDS"]
    if c.get("TCC_HIT_sum", 0.0) + c.get("TCC_MISS_sum", 0.0) > 0:
        out["l2_hit_rate"] = c.get("TCC_HIT_sum", 0.0) / (c.get("TCC_HIT_sum", 0.0) + c.get("TCC_MISS_sum", 0.0))
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    t = sub.add_parser("traffic")
    for k in ("read", "write", "copy_read", "copy_write"):
        t.add_argument("--" + k.replace("_", "-"), required=True)
    t.add_argument("--kernel", required=True, help="regex on the kernel name")
    t.add_argument("--stage", required=True, choices=sorted(STAGE_SOURCES))
    t.add_argument("--workload", required=True)
    t.add_argument("--copy-bytes", type=float, default=float(1 << 30))
    t.add_argument("--json")
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--kernel", action="append", required=True, help="regex on the kernel name")
    a = ap.parse_args(argv)

    if a.cmd == "stats":
        print(f"{'kernel':34s} {'calls':>6s} {'total_us':>11s} {'avg_us':>10s} {'pct':>7s}")
        for n, calls, tot, avg, pct in stats(a.dir):
            print(f"{n:34s} {calls:6d} {tot:11.1f} {avg:10.2f} {pct:7.2f}")
        return 0
    if a.cmd == "counters":
        for kre in a.kernel:
            r = counters(a.dirs, kre)
            print(f"== /{kre}/ (means per dispatch)")
            for k, v in r.items():
                if k != "raw":
                    print(f"  {k:36s} {v:.4g}")
            for k, v in sorted(r["raw"].items()):
                print(f"  {k:36s} {v:.6g}")
        return 0
    rec = traffic(a)
    print(json.dumps(rec, indent=1))
    if a.json:
        with open(a.json, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
