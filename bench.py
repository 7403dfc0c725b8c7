#!/usr/bin/env python3
"""Benchmark of the block-sparse attention forward on one MI355X.

One step = one full forward over one batch of resident synthetic inputs:
block_pool -> coarse_select (coarse scores and top-k in one kernel) ->
block-gather sparse_flash_fwd (gather_index, attention, gather_combine).
Prints ONE JSON line: forward tokens/s (batch * n / step time), effective
TFLOP/s, the roofline of the dominant kernel (timed with HIP events on the
launch stream inside this run), the bound and fraction of every stage
(`stage_rooflines`, longest first), the step against the sum of the stages'
ideal times (`path_roofline`), the median and minimum of single steps
run after a cache-flushing 1 GiB write (`cold`), and the fp64 CPU oracle's
throughput on a bounded sample of the same workload.

With --pass backward a step is one bsa_backward (dq, dk, dv of the fine stage
for the selection, output and lse of one bsa_forward_train made before the
timed region) and the line reports backward tokens/s.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--pass forward|backward]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "fwd tokens/s and effective TFLOP/s at N=32k,H=8,D=64,B=64,k=16; % roofline"
METRIC_BWD = "bwd tokens/s (fine-stage dq, dk, dv; selection fixed) and effective TFLOP/s; % roofline"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3}
def visible_pairs(w: W.Workload) -> int:
    """Closed form of the (query, key) pairs the fine stage visits."""
    nb = w.nb
    if not w.causal:
        return w.bh * w.n * min(w.topk, nb) * w.block
    i = np.arange(w.n, dtype=np.int64)
    qb = i // w.block
    keff = np.minimum(w.topk, qb + 1)
    return int(w.bh * ((keff - 1) * w.block + (i % w.block) + 1).sum())


def candidate_pairs(w: W.Workload) -> int:
    if not w.causal:
        return w.bh * w.n * w.nb
    i = np.arange(w.n, dtype=np.int64)
    return int(w.bh * (i // w.block + 1).sum())


def stage_work(w: W.Workload):
    """Algorithmic work per launch of each kernel over the whole problem:
    (flops, bytes).  Bytes count each compulsory read/write once; a kernel's
    roofline bound is whichever of the two takes longer at the MI355X peaks."""
    s = 2 if w.dtype == "bf16" else 4
    qkv = w.bh * w.n * w.d * s
    repr_b = w.bh * w.nb * w.d * 4
    cand = candidate_pairs(w)
    panel = cand * 4
    idx = w.bh * w.n * w.topk * 4
    fine_flops = 4 * w.d * visible_pairs(w)
    sel_pairs = w.bh * w.n * min(w.topk, w.nb) if not w.causal else None
    if sel_pairs is None:
        i = np.arange(w.n, dtype=np.int64)
        sel_pairs = int(w.bh * np.minimum(w.topk, i // w.block + 1).sum())
    partial = sel_pairs * w.d * (2 if w.dtype == "bf16" else 4)
    out_b = w.bh * w.n * w.d * 4
    rows = w.bh * w.n
    dq_rows = sel_pairs * w.d * s  # per-pair dq rows: bf16 (bf16 inputs) or fp32
    return {
        "block_pool": (0, qkv + repr_b),
        "coarse_score": (2 * w.d * cand, qkv + repr_b + panel),
        "topk_select": (0, panel + idx),
        # fused scoring + selection: q and the representatives in, indices out
        "coarse_select": (2 * w.d * cand, qkv + repr_b + idx),
        # block-gather attention kernel: reads Q, K, V once, writes the partials
        "sparse_flash_fwd": (fine_flops, 3 * qkv + idx + partial),
        "gather_index": (0, 2 * idx + 3 * sel_pairs * 4),
        "gather_combine": (0, partial + idx + out_b),
        # backward: out, dout and lse in; per-row (lse, delta) and (bf16 inputs) bf16 dout out
        "bwd_prep": (0, 2 * out_b + rows * (4 + 8) + (qkv if w.dtype == "bf16" else 0)),
        "bwd_index": (0, 2 * idx + 3 * sel_pairs * 4),
        # S, dP, dQ, dK, dV: five products per visible (query, key) pair; reads
        # Q, K, V, dout (bf16 copy for bf16 inputs) and the row statistics
        # once, writes the per-pair dq rows
        "bwd_pairs": (10 * w.d * visible_pairs(w),
                      3 * qkv + (qkv if w.dtype == "bf16" else out_b) + rows * 8 + dq_rows),
        # per-pair dq rows in; dq, dk, dv out
        "bwd_reduce": (0, dq_rows + idx + 3 * out_b),
    }


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    from content_dependent_block_amd.rocprof_summary import source_sha
    p = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        c = json.load(f)
    if c.get("source_sha") != source_sha(kernel):
        return None
    return c.get("hbm_bytes_per_launch")


def cpu_baseline(w: W.Workload, inp, positions: int):
    import oracle
    n_pos = min(positions, w.n)
    pos = np.linspace(0, w.n - 1, n_pos).astype(np.int64)
    rows = (np.arange(w.bh, dtype=np.int64)[:, None] * w.n + pos[None, :]).ravel()
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    t0 = time.perf_counter()
    oracle.forward(inp.q, inp.k, inp.v, w.block, w.topk, w.causal, w.scale, rows)
    dt = time.perf_counter() - t0
    return {"value": n_pos * w.batch / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_pos} of {w.n} query positions (evenly spaced) x all {w.bh} heads; "
                      f"pool + coarse scores + top-k + two-pass softmax attention in fp64; "
                      f"{dt:.2f} s wall"}


def cpu_baseline_backward(w: W.Workload, inp, dout):
    """The oracle's backward over one head (all its rows and key blocks),
    scaled to all heads."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    r = oracle.pool(inp.k[:, :1], w.block)
    sc = oracle.scores(inp.q[:, :1], r, w.block)
    idx, _, _ = oracle.topk(sc, w.n, w.block, w.topk, w.causal)
    t0 = time.perf_counter()
    oracle.attend_backward(inp.q[:, :1], inp.k[:, :1], inp.v[:, :1], dout[:, :1], idx, w.block,
                           w.causal, w.scale)
    dt = time.perf_counter() - t0
    return {"value": w.n * w.batch / (dt * w.heads), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"head 0 of {w.heads} (all {w.n} rows, all key blocks): dq, dk, dv, lse in "
                      f"fp64 on the oracle's own selection; {dt:.2f} s wall, scaled to {w.heads} heads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=W.HEADLINE, choices=sorted(W.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-positions", type=int, default=32768)
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="extra steps timed one by one after a cache-flushing 1 GiB write (0 = none)")
    ap.add_argument("--fine-strategy", choices=["block_gather", "query_tile"], default="block_gather")
    ap.add_argument("--select-strategy", choices=["fused", "panel"], default="fused")
    ap.add_argument("--panel-chunk-mb", type=int, default=0, help="coarse-score panel chunk (0 = default)")
    ap.add_argument("--fine-chunk-mb", type=int, default=0, help="block-gather partial chunk (0 = default)")
    ap.add_argument("--pass", dest="which", choices=["forward", "backward"], default="forward")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB -> 1 GiB device copy (3 times), the reference "
                         "for scaling the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the library runs on one GPU; there is no multi-GPU mode "
              "(heads would shard across GPUs with no communication).", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": src.numel() * 4,
                          "copy_calibration_bytes_written": dst.numel() * 4, "launches": 3}))
        return

    import content_dependent_block_amd as m

    w = W.WORKLOADS[args.workload]
    if w.static:
        raise SystemExit("bench.py times the dynamic two-stage forward; pick a dynamic workload")
    inp = W.generate(w)
    dev = torch.device("cuda:0")
    if w.dtype == "bf16":
        q, k, v = (torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)
                   for b in (inp.q_bits, inp.k_bits, inp.v_bits))
    else:
        q, k, v = (torch.from_numpy(x).to(dev) for x in (inp.q, inp.k, inp.v))
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    idx = torch.empty(q.shape[:3] + (w.topk,), dtype=torch.int32, device=dev)
    lib = m.BlockSparseAttention(0)
    h = lib.handle
    m.bsa_set_option(h, m.BSA_OPT_FINE_STRATEGY,
                     m.BSA_FINE_BLOCK_GATHER if args.fine_strategy == "block_gather" else m.BSA_FINE_QUERY_TILE)
    m.bsa_set_option(h, m.BSA_OPT_SELECT_STRATEGY,
                     m.BSA_SELECT_FUSED if args.select_strategy == "fused" else m.BSA_SELECT_PANEL)
    if args.panel_chunk_mb:
        m.bsa_set_option(h, m.BSA_OPT_PANEL_CHUNK_BYTES, args.panel_chunk_mb << 20)
    if args.fine_chunk_mb:
        m.bsa_set_option(h, m.BSA_OPT_FINE_CHUNK_BYTES, args.fine_chunk_mb << 20)

    if args.which == "forward":
        def step():
            m.bsa_forward(h, q, k, v, out, idx, topk=w.topk, scale=w.scale, causal=w.causal)
    else:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        m.bsa_forward_train(h, q, k, v, out, idx, lse, topk=w.topk, scale=w.scale, causal=w.causal)
        dout_np = W.grad_output(q.shape, w.seed)
        dout = torch.from_numpy(dout_np).to(dev)
        dq, dk, dv = (torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in range(3))

        def step():
            m.bsa_backward(h, q, k, v, out, dout, idx, lse, dq, dk, dv, scale=w.scale, causal=w.causal)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps

    # Cold steps (after the timed region, not part of `value`): before each
    # step a 1 GiB scratch buffer is written, which evicts the inputs from
    # the 256 MB Infinity Cache; each step is timed alone with HIP events.
    cold = None
    if args.cold_steps > 0:
        scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        times = []
        for i in range(args.cold_steps):
            scratch.fill_(float(i))
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record(stream)
            step()
            c1.record(stream)
            torch.cuda.synchronize()
            times.append(c0.elapsed_time(c1))
        del scratch
        cold = {"steps": args.cold_steps, "ms_median": round(float(np.median(times)), 5),
                "ms_min": round(float(np.min(times)), 5),
                "flush": "1 GiB scratch written before each step"}

    # Second pass: per-kernel HIP events on the launch stream.
    m.bsa_profile_read(h, reset=True)
    m.bsa_profile_enable(h, True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms, launches = m.bsa_profile_read(h, reset=True)
    m.bsa_profile_enable(h, False)
    per_step = {name: ms[i] / args.steps for i, name in enumerate(m.STAGE_NAMES) if launches[i]}
    per_launch = {name: ms[i] / launches[i] for i, name in enumerate(m.STAGE_NAMES) if launches[i]}
    launches_per_step = {name: launches[i] // args.steps for i, name in enumerate(m.STAGE_NAMES)
                         if launches[i]}

    work = stage_work(w)

    def stage_roofline(name):
        """The roofline of one stage: its algorithmic flops (MFMA-bound) or
        bytes (HBM-bound) per launch over its average launch time; the bound
        is the resource whose peak the algorithmic work would take longer on."""
        flops, nbytes = work[name]
        t_launch = per_launch[name] * 1e-3
        n_launch = launches_per_step[name]
        t_mfma = flops / (MFMA_PEAK_TFLOPS[w.dtype] * 1e12)
        t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
        if t_mfma >= t_hbm:
            achieved, peak, unit = flops / n_launch / t_launch / 1e12, MFMA_PEAK_TFLOPS[w.dtype], "TFLOP/s"
        else:
            achieved, peak, unit = nbytes / n_launch / t_launch / 1e9, HBM_PEAK_GBS, "GB/s"
        return {"bound": "mfma" if t_mfma >= t_hbm else "hbm", "achieved": round(achieved, 3), "peak": peak,
                "unit": unit, "frac": round(achieved / peak, 5)}

    dom = max(per_step, key=per_step.get)
    roofline = dict(stage_roofline(dom), traffic=measured_traffic(dom, w.name), kernel=dom,
                    avg_launch_ms=round(per_launch[dom], 5), launches_per_step=launches_per_step[dom])
    # the whole step against the sum of every stage's ideal time (the longer of
    # its algorithmic flops at the MFMA peak and its algorithmic bytes at the
    # HBM peak)
    ideal_ms = sum(max(work[k_][0] / (MFMA_PEAK_TFLOPS[w.dtype] * 1e12), work[k_][1] / (HBM_PEAK_GBS * 1e9))
                   for k_ in per_step) * 1e3
    path_roofline = {"ideal_ms": round(ideal_ms, 5), "frac": round(ideal_ms / ms_per_step, 5)}
    if args.which == "forward":
        # strict: the method's three steps with compulsory bytes only (Q, K, V
        # read once, O written, representatives and indices written and read
        # once; no score panel, no split-softmax partials)
        s_ = 2 if w.dtype == "bf16" else 4
        qkv_b = w.bh * w.n * w.d * s_
        repr_b = w.bh * w.nb * w.d * 4
        idx_b = w.bh * w.n * w.topk * 4
        out_b = w.bh * w.n * w.d * 4
        peak_f = MFMA_PEAK_TFLOPS[w.dtype] * 1e12
        peak_b = HBM_PEAK_GBS * 1e9
        strict_s = (max(0.0, (qkv_b + repr_b) / peak_b)
                    + max(work["coarse_select"][0] / peak_f, (qkv_b + repr_b + idx_b) / peak_b)
                    + max(4 * w.d * visible_pairs(w) / peak_f, (3 * qkv_b + idx_b + out_b) / peak_b))
        path_roofline["strict_ideal_ms"] = round(strict_s * 1e3, 5)
        path_roofline["strict_frac"] = round(strict_s * 1e3 / ms_per_step, 5)
    # every stage's bound and fraction, longest first (the first is `roofline`)
    stage_rooflines = {k_: {f: stage_roofline(k_)[f] for f in ("bound", "achieved", "unit", "frac")}
                       for k_ in sorted(per_step, key=per_step.get, reverse=True)}

    total_flops = sum(work[k_][0] for k_ in per_step)  # matmul-only: coarse + fine, stages that ran
    tokens = w.batch * w.n
    result = {
        "metric": METRIC if args.which == "forward" else METRIC_BWD,
        "value": round(tokens / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded N(0,1) q/k/v plus per-block key offsets N(0,0.5^2), "
                "rounded to bf16 (no dataset)" if w.key_offsets else "synthetic: seeded N(0,1)",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "n": w.n, "d": w.d,
                   "block": w.block, "topk": w.topk, "causal": w.causal,
                   "select_strategy": args.select_strategy, "fine_strategy": args.fine_strategy,
                   "panel_chunk_mb": args.panel_chunk_mb or 128, "fine_chunk_mb": args.fine_chunk_mb or 1024,
                   "pass": args.which},
        "effective_tflops": round(total_flops / (ms_per_step * 1e-3) / 1e12, 3),
        "algorithmic_gflop": round(total_flops / 1e9, 3),
        "stage_ms_per_step": {k_: round(v_, 5) for k_, v_ in per_step.items()},
        "roofline": roofline,
        "stage_rooflines": stage_rooflines,
        "path_roofline": path_roofline,
    }
    if cold is not None:
        result["cold"] = cold
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = (cpu_baseline(w, inp, args.cpu_positions) if args.which == "forward"
                                  else cpu_baseline_backward(w, inp, dout_np))
    lib.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
