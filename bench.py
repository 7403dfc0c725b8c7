#!/usr/bin/env python3
"""Benchmark of the block-sparse attention forward on one MI355X.

One step = one full forward over one batch of resident synthetic inputs:
block_pool -> coarse_select (coarse scores and top-k in one kernel) ->
block-gather sparse_flash_fwd (gather_index, attention, gather_combine); for
the static workload one bsa_forward_static over its tile list.

Timing protocol: W untimed warm-up steps; then K cold steps, each after a
1 GiB scratch write that evicts the inputs from the 256 MB Infinity Cache,
followed by a read of the same buffer, and timed with HIP events on the
launch stream.  The step is queued behind the flush (write, read, start
event, step, end event, then a device synchronisation), so the host has
issued the step's launches before its start event fires, as in a stream of
back-to-back calls.  The read leaves the cache holding clean lines; after
the write alone up to 256 MB of dirty lines remain, whose write-back the
next step would pay for (--cache-check measures every case on a plain
tensor read).  `value` is tokens/s at the MEDIAN cold step; beside it the
line reports the warm figure (K steps back to back), the cold median with
a device synchronisation before each start event (the host's issue of the
first kernel then counts too), and the cold median after the write alone.  Per-kernel times come from
another queued cold pass with per-stage HIP events on the launch stream
(the roofline of the dominant kernel is computed from those).

Prints ONE JSON line: the headline workload's tokens/s, effective TFLOP/s,
the roofline of the dominant kernel, every stage's bound and fraction, the
step against the sum of the stages' ideal times, the fp64 CPU oracle's
throughput on the host cores (plus a one-thread time of the small workload),
and (unless --only) the same timings for every other workload.

With --pass backward a step is one bsa_backward (dq, dk, dv of the fine stage
for the selection, output and lse of one bsa_forward_train made before the
timed region) and the line reports backward tokens/s.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--only]
                    [--no-cpu-baseline] [--pass forward|backward]
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
    if w.static:
        return static_visible_pairs(w)
    nb = w.nb
    if not w.causal:
        return w.bh * w.n * min(w.topk, nb) * w.block
    i = np.arange(w.n, dtype=np.int64)
    qb = i // w.block
    keff = np.minimum(w.topk, qb + 1)
    return int(w.bh * ((keff - 1) * w.block + (i % w.block) + 1).sum())


def static_visible_pairs(w: W.Workload) -> int:
    """Pairs with |i - j| <= window or j mod stride == 0, counted per row."""
    i = np.arange(w.n, dtype=np.int64)
    lo = np.maximum(0, i - w.window)
    hi = np.minimum(w.n - 1, i + w.window)
    band = hi - lo + 1
    glob_all = (w.n - 1) // w.stride + 1
    # global keys inside the band are counted once
    glob_in_band = hi // w.stride - (lo - 1) // w.stride
    glob_in_band = np.where(lo == 0, hi // w.stride + 1, glob_in_band)
    return int(w.bh * (band + glob_all - glob_in_band).sum())


def candidate_pairs(w: W.Workload) -> int:
    if not w.causal:
        return w.bh * w.n * w.nb
    i = np.arange(w.n, dtype=np.int64)
    return int(w.bh * (i // w.block + 1).sum())


def stage_work(w: W.Workload, nnz: int = 0):
    """Algorithmic work per step of each kernel over the whole problem:
    (flops, bytes).  Only the method's own work counts: the matmul flops of
    scoring and of attention over the visible pairs, and each compulsory
    tensor (Q, K, V, representatives, indices, output; for the backward dout,
    out, lse and the gradients) read or written once.  Buffers that are this
    implementation's choice (score panel, bucket lists, per-pair partial and
    dq rows) count nothing, so a kernel's fraction says how far it is from the
    method's bound.  A kernel's roofline bound is whichever of flops and bytes
    takes longer at the MI355X peaks."""
    s = 2 if w.dtype == "bf16" else 4
    qkv = w.bh * w.n * w.d * s
    out_b = w.bh * w.n * w.d * 4
    fine_flops = 4 * w.d * visible_pairs(w)
    if w.static:
        lst = nnz * 4 + nnz * 64 * 8  # key-tile ids and row masks
        return {"sparse_flash_fwd": (fine_flops, 3 * qkv + lst + out_b),
                "static_combine": (0, 0)}
    repr_b = w.bh * w.nb * w.d * 4
    cand = candidate_pairs(w)
    idx = w.bh * w.n * w.topk * 4
    rows = w.bh * w.n
    return {
        "block_pool": (0, qkv + repr_b),
        "coarse_score": (2 * w.d * cand, qkv + repr_b),
        "topk_select": (0, idx),
        # fused scoring + selection: q and the representatives in, indices out
        "coarse_select": (2 * w.d * cand, qkv + repr_b + idx),
        # block-gather attention: the fine flops; Q, K, V and the indices read once
        "sparse_flash_fwd": (fine_flops, 3 * qkv + idx),
        "gather_index": (0, 0),
        # the merge writes the output once
        "gather_combine": (0, out_b),
        # backward: out, dout and lse read once
        "bwd_prep": (0, 2 * out_b + rows * 4),
        "bwd_index": (0, 0),
        # S, dP, dQ, dK, dV: five products per visible (query, key) pair; Q, K,
        # V and the indices read once, dk and dv written once
        "bwd_pairs": (10 * w.d * visible_pairs(w), 3 * qkv + idx + 2 * out_b),
        # dq written once
        "bwd_reduce": (0, out_b),
        "ragged_copy": (0, 0),
    }


def strict_ideal_s(w: W.Workload, nnz: int = 0) -> float:
    """The method's steps with compulsory bytes only: Q, K, V read once, O
    written, representatives and indices written and read once; no score
    panel and no split-softmax partials."""
    peak_f = MFMA_PEAK_TFLOPS[w.dtype] * 1e12
    peak_b = HBM_PEAK_GBS * 1e9
    s_ = 2 if w.dtype == "bf16" else 4
    qkv_b = w.bh * w.n * w.d * s_
    out_b = w.bh * w.n * w.d * 4
    fine_f = 4 * w.d * visible_pairs(w)
    if w.static:
        return max(fine_f / peak_f, (3 * qkv_b + out_b + nnz * (4 + 512)) / peak_b)
    repr_b = w.bh * w.nb * w.d * 4
    idx_b = w.bh * w.n * w.topk * 4
    return ((qkv_b + repr_b) / peak_b
            + max(2 * w.d * candidate_pairs(w) / peak_f, (qkv_b + repr_b + idx_b) / peak_b)
            + max(fine_f / peak_f, (3 * qkv_b + idx_b + out_b) / peak_b))


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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w: W.Workload, inp, positions: int, static_mask=None):
    """The fp64 oracle on the host cores over a bounded sample of the same
    workload (all heads, evenly spaced query positions), plus the whole
    small workload on one thread."""
    import oracle
    threads = oracle.threads()
    n_pos = min(positions, w.n)
    pos = np.linspace(0, w.n - 1, n_pos).astype(np.int64)
    rows = (np.arange(w.bh, dtype=np.int64)[:, None] * w.n + pos[None, :]).ravel()
    t0 = time.perf_counter()
    if w.static:
        oracle.attend_mask(inp.q, inp.k, inp.v, static_mask, w.scale, rows)
        what = "masked softmax attention in fp64"
    else:
        oracle.forward(inp.q, inp.k, inp.v, w.block, w.topk, w.causal, w.scale, rows)
        what = "pool + coarse scores + top-k + two-pass softmax attention in fp64"
    dt = time.perf_counter() - t0
    res = {"value": round(n_pos * w.batch / dt, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{n_pos} of {w.n} query positions (evenly spaced) x all {w.bh} heads; {what}; "
                     f"{dt:.2f} s wall", "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}
    # the small workload in full on one thread
    ws = W.WORKLOADS[W.SMALL]
    si = W.generate(ws)
    before = oracle.set_threads(1)
    try:
        t0 = time.perf_counter()
        oracle.forward(si.q, si.k, si.v, ws.block, ws.topk, ws.causal, ws.scale)
        dt1 = time.perf_counter() - t0
    finally:
        oracle.set_threads(before)
    res["one_thread_small"] = {"workload": ws.name, "seconds": round(dt1, 4),
                               "tokens_per_s": round(ws.n * ws.batch / dt1, 1), "cores": 1}
    return res


def cpu_baseline_backward(w: W.Workload, inp, dout):
    """The oracle's backward over one head (all its rows and key blocks),
    scaled to all heads."""
    import oracle
    threads = oracle.threads()
    r = oracle.pool(inp.k[:, :1], w.block)
    sc = oracle.scores(inp.q[:, :1], r, w.block)
    idx, _, _ = oracle.topk(sc, w.n, w.block, w.topk, w.causal)
    t0 = time.perf_counter()
    oracle.attend_backward(inp.q[:, :1], inp.k[:, :1], inp.v[:, :1], dout[:, :1], idx, w.block,
                           w.causal, w.scale)
    dt = time.perf_counter() - t0
    return {"value": round(w.n * w.batch / (dt * w.heads), 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"head 0 of {w.heads} (all {w.n} rows, all key blocks): dq, dk, dv, lse in "
                      f"fp64 on the oracle's own selection; {dt:.2f} s wall, scaled to {w.heads} heads"}


def union_stats(idx, w: W.Workload):
    """For query tiles of 16, 32 and 64 rows: the mean number of distinct
    blocks the tile's rows selected (the blocks a query-tile union visits),
    and the flops a union kernel issues when every row of the tile meets
    every block of the union (S = Q K^T and O = P V over 64 keys each)."""
    import torch
    bh, n, k = idx.shape[0] * idx.shape[1], idx.shape[2], idx.shape[3]
    sel = idx.reshape(bh, n, k).long()
    out = {}
    for tq in (16, 32, 64):
        t = sel.reshape(bh, n // tq, tq * k)
        hit = torch.zeros((bh, n // tq, w.nb + 1), dtype=torch.bool, device=idx.device)
        hit.scatter_(2, torch.where(t >= 0, t, torch.full_like(t, w.nb)), True)
        per_tile = hit[:, :, :w.nb].sum(dim=2).double()
        out[str(tq)] = {"blocks_per_tile": round(float(per_tile.mean()), 2),
                        "issued_tflop": round(float(per_tile.sum()) * tq * 64 * 4 * w.d / 1e12, 4)}
    return out


class Runner:
    """Inputs of one workload resident on the device and its step function."""

    def __init__(self, m, lib, w: W.Workload, which: str, args):
        import torch
        self.torch, self.m, self.lib, self.w = torch, m, lib, w
        self.inp = W.generate(w)
        dev = torch.device("cuda:0")
        inp = self.inp
        if w.dtype == "bf16":
            q, k, v = (torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)
                       for b in (inp.q_bits, inp.k_bits, inp.v_bits))
        else:
            q, k, v = (torch.from_numpy(x).to(dev) for x in (inp.q, inp.k, inp.v))
        out = torch.empty(q.shape, dtype=torch.float32, device=dev)
        h = lib.handle
        self.nnz = 0
        self.mask = None
        self.tiles = None
        self.dout_np = None
        self.idx = None
        if w.static:
            rp, col, rm = m.bsa_tiles_window_stride(w.n, w.window, w.stride)
            self.nnz = int(col.size)
            self.tiles = m.bsa_tiles_create(h, w.n, rp, col, rm)
            tiles = self.tiles

            def step():
                m.bsa_forward_static(h, q, k, v, out, tiles, scale=w.scale)
        elif which == "forward":
            idx = torch.empty(q.shape[:3] + (w.topk,), dtype=torch.int32, device=dev)

            def step():
                m.bsa_forward(h, q, k, v, out, idx, topk=w.topk, scale=w.scale, causal=w.causal)
            self.idx = idx
        else:
            idx = torch.empty(q.shape[:3] + (w.topk,), dtype=torch.int32, device=dev)
            lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
            m.bsa_forward_train(h, q, k, v, out, idx, lse, topk=w.topk, scale=w.scale, causal=w.causal)
            self.dout_np = W.grad_output(q.shape, w.seed)
            dout = torch.from_numpy(self.dout_np).to(dev)
            dq, dk, dv = (torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in range(3))

            def step():
                m.bsa_backward(h, q, k, v, out, dout, idx, lse, dq, dk, dv, scale=w.scale, causal=w.causal)
        self.step = step
        self.stream = torch.cuda.current_stream(dev)
        self.tensors = [q, k, v, out]

    def close(self):
        if self.tiles is not None:
            self.tiles.close()
        self.tensors = []

    def warm(self, steps):
        """Mean milliseconds of `steps` back-to-back steps."""
        torch = self.torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(self.stream)
        for _ in range(steps):
            self.step()
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def cold(self, steps, scratch, profile=False, synced=False, flush="write_read"):
        """Milliseconds of each of `steps` steps, each after a 1 GiB scratch
        write and a read of the same buffer (flush="write": the write alone)
        on the same stream; with profile, also the per-stage HIP-event times.
        synced: wait for the flush before issuing the step, so its time also
        holds the host's issue of the first kernel."""
        torch, m, h = self.torch, self.m, self.lib.handle
        if profile:
            m.bsa_profile_read(h, reset=True)
            m.bsa_profile_enable(h, True)
        times = []
        for i in range(steps):
            scratch.fill_(float(i))
            if flush == "write_read":
                torch.sum(scratch)
            if synced:
                torch.cuda.synchronize()
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record(self.stream)
            self.step()
            c1.record(self.stream)
            torch.cuda.synchronize()
            times.append(c0.elapsed_time(c1))
        stages = None
        if profile:
            ms, launches = m.bsa_profile_read(h, reset=True)
            m.bsa_profile_enable(h, False)
            stages = {name: (ms[i], launches[i]) for i, name in enumerate(m.STAGE_NAMES) if launches[i]}
        return times, stages


def stage_roofline(w, work, name, per_launch_ms, launches_per_step):
    """The roofline of one stage: its algorithmic flops (MFMA-bound) or bytes
    (HBM-bound) per launch over its average launch time; the bound is the
    resource whose peak the algorithmic work would take longer on."""
    flops, nbytes = work[name]
    t_launch = per_launch_ms * 1e-3
    t_mfma = flops / (MFMA_PEAK_TFLOPS[w.dtype] * 1e12)
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    if t_mfma >= t_hbm:
        achieved, peak, unit = flops / launches_per_step / t_launch / 1e12, MFMA_PEAK_TFLOPS[w.dtype], "TFLOP/s"
    else:
        achieved, peak, unit = nbytes / launches_per_step / t_launch / 1e9, HBM_PEAK_GBS, "GB/s"
    return {"bound": "mfma" if t_mfma >= t_hbm else "hbm", "achieved": round(achieved, 3), "peak": peak,
            "unit": unit, "frac": round(achieved / peak, 5)}


def cache_check(torch, reps=15):
    """Median microseconds of one read of a 200 MB tensor x (it fits the
    256 MB Infinity Cache), taken right after x was read once more and then
    after nothing, a 1 GiB read, a 1 GiB write, that write followed by a
    read of the same buffer (the cold steps' flush), or a 2 GiB read.  Equal
    times after a 1 GiB and a 2 GiB read mean a 1 GiB read evicts x; a
    longer time after the write alone is the write-back of its dirty lines,
    paid by the read that follows it."""
    dev = "cuda:0"
    x = torch.ones(50 << 20, dtype=torch.float32, device=dev)
    a1 = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    a2 = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    flushes = {"none": lambda i: None, "read_1gib": lambda i: torch.sum(a1),
               "write_1gib": lambda i: a1.fill_(float(i)),
               "write_then_read_1gib": lambda i: (a1.fill_(float(i)), torch.sum(a1)),
               "read_2gib": lambda i: (torch.sum(a1), torch.sum(a2))}
    res = {"x_bytes": x.numel() * 4}
    for name, fl in flushes.items():
        ts = []
        for i in range(reps):
            torch.sum(x)
            fl(i)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            torch.sum(x)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        res[f"read_x_after_{name}_us"] = round(float(np.median(ts)), 1)
    return res


def measure(r: Runner, args, scratch, steps, warmup):
    """Warm-up, cold steps (the value), warm steps, cold per-stage times."""
    w = r.w
    for _ in range(warmup):
        r.step()
    r.torch.cuda.synchronize()
    cold_t, _ = r.cold(steps, scratch)
    synced_t, _ = r.cold(steps, scratch, synced=True)
    write_t, _ = r.cold(steps, scratch, flush="write")
    warm_ms = r.warm(steps)
    _, stages = r.cold(steps, scratch, profile=True)
    per_step = {k: v[0] / steps for k, v in stages.items()}
    per_launch = {k: v[0] / v[1] for k, v in stages.items()}
    lps = {k: v[1] // steps for k, v in stages.items()}
    work = stage_work(w, r.nnz)
    ms_med = float(np.median(cold_t))
    tokens = w.batch * w.n
    total_flops = sum(work[k][0] for k in per_step if k in work)
    res = {
        "ms_cold_median": round(ms_med, 5), "ms_cold_min": round(float(np.min(cold_t)), 5),
        "ms_cold_mean": round(float(np.mean(cold_t)), 5), "ms_warm": round(warm_ms, 5),
        "ms_cold_synced_median": round(float(np.median(synced_t)), 5),
        "ms_cold_write_flush_median": round(float(np.median(write_t)), 5),
        "tokens_per_s": round(tokens / (ms_med * 1e-3), 1),
        "tokens_per_s_warm": round(tokens / (warm_ms * 1e-3), 1),
        "effective_tflops": round(total_flops / (ms_med * 1e-3) / 1e12, 3),
        "algorithmic_gflop": round(total_flops / 1e9, 4),
        "stage_ms_per_step": {k: round(v, 5) for k, v in per_step.items()},
    }
    known = [k for k in per_step if k in work and (work[k][0] or work[k][1])]
    dom = max(known, key=per_step.get)
    res["roofline"] = dict(stage_roofline(w, work, dom, per_launch[dom], lps[dom]),
                           traffic=measured_traffic(dom, w.name) if dom in _TRAFFIC_STAGES else None,
                           kernel=dom, avg_launch_ms=round(per_launch[dom], 5), launches_per_step=lps[dom])
    res["stage_rooflines"] = {k: {f: stage_roofline(w, work, k, per_launch[k], lps[k])[f]
                                  for f in ("bound", "achieved", "unit", "frac")}
                              for k in sorted(known, key=per_step.get, reverse=True)}
    ideal_ms = sum(max(work[k][0] / (MFMA_PEAK_TFLOPS[w.dtype] * 1e12), work[k][1] / (HBM_PEAK_GBS * 1e9))
                   for k in known) * 1e3
    res["path_roofline"] = {"ideal_ms": round(ideal_ms, 5), "frac": round(ideal_ms / ms_med, 5)}
    if args.which == "forward":
        # The method page's own FLOP convention: the matmul flops plus 5 per
        # attention score element (its dense and sparse totals both follow
        # from this); the matmul-only figure above stays the primary one.
        page_flops = total_flops + 5 * visible_pairs(w)
        res["page_convention"] = {"gflop": round(page_flops / 1e9, 4),
                                  "tflops": round(page_flops / (ms_med * 1e-3) / 1e12, 3)}
        if not w.static and "sparse_flash_fwd" in per_step:
            # The fine stage against HBM bandwidth over per-query gathered
            # bytes (every visible pair's key and value rows read once per
            # query): a sanity figure that exceeds 1 whenever caches reuse
            # key blocks across queries, which block-gather is built on.
            gathered = visible_pairs(w) * 2 * w.d * (2 if w.dtype == "bf16" else 4)
            ideal = gathered / (HBM_PEAK_GBS * 1e9) * 1e3
            res["gather_r2"] = {"per_query_gather_gb": round(gathered / 1e9, 3), "ideal_ms": round(ideal, 4),
                                "attention_ms": round(per_step["sparse_flash_fwd"], 5),
                                "frac": round(ideal / per_step["sparse_flash_fwd"], 3)}
        strict_ms = strict_ideal_s(w, r.nnz) * 1e3
        res["path_roofline"]["strict_ideal_ms"] = round(strict_ms, 5)
        res["path_roofline"]["strict_frac"] = round(strict_ms / ms_med, 5)
    return res


_TRAFFIC_STAGES = ("block_pool", "coarse_score", "topk_select", "coarse_select", "sparse_flash_fwd",
                   "gather_index", "gather_combine", "bwd_prep", "bwd_index", "bwd_pairs", "bwd_reduce")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=W.HEADLINE, choices=sorted(W.WORKLOADS))
    ap.add_argument("--only", action="store_true", help="time the chosen workload only")
    ap.add_argument("--other-steps", type=int, default=20, help="cold steps for each other workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-positions", type=int, default=32768)
    ap.add_argument("--fine-strategy", choices=["block_gather", "query_tile", "per_query"], default="block_gather")
    ap.add_argument("--union-rows", type=int, choices=[16, 32, 64], default=64,
                    help="query-tile rows of the query_tile fine strategy")
    ap.add_argument("--union-stats", action="store_true",
                    help="report the query-tile unions of the selection (16, 32 and 64 rows)")
    ap.add_argument("--select-strategy", choices=["fused", "panel"], default="fused")
    ap.add_argument("--panel-chunk-mb", type=int, default=0, help="coarse-score panel chunk (0 = default)")
    ap.add_argument("--fine-chunk-mb", type=int, default=0, help="block-gather partial chunk (0 = default)")
    ap.add_argument("--static-item-tiles", type=int, default=0, help="static work-item size (0 = per call)")
    ap.add_argument("--pass", dest="which", choices=["forward", "backward"], default="forward")
    ap.add_argument("--cache-check", action="store_true",
                    help="run only the check of the cold-step flush: a 200 MB tensor read after no "
                         "flush, a 1 GiB read, a 1 GiB write, that write and a read of it, a 2 GiB read")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB -> 1 GiB device copy (3 times), the reference "
                         "for scaling the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the library runs on one GPU; there is no multi-GPU mode "
              "(heads would shard across GPUs with no communication).", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.cache_check:
        print(json.dumps(cache_check(torch)))
        return

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
    lib = m.BlockSparseAttention(0)
    h = lib.handle
    m.bsa_set_option(h, m.BSA_OPT_FINE_STRATEGY,
                     {"block_gather": m.BSA_FINE_BLOCK_GATHER, "query_tile": m.BSA_FINE_QUERY_TILE,
                      "per_query": m.BSA_FINE_PER_QUERY}[args.fine_strategy])
    m.bsa_set_option(h, m.BSA_OPT_UNION_ROWS, args.union_rows)
    m.bsa_set_option(h, m.BSA_OPT_SELECT_STRATEGY,
                     m.BSA_SELECT_FUSED if args.select_strategy == "fused" else m.BSA_SELECT_PANEL)
    if args.panel_chunk_mb:
        m.bsa_set_option(h, m.BSA_OPT_PANEL_CHUNK_BYTES, args.panel_chunk_mb << 20)
    if args.fine_chunk_mb:
        m.bsa_set_option(h, m.BSA_OPT_FINE_CHUNK_BYTES, args.fine_chunk_mb << 20)
    m.bsa_set_option(h, m.BSA_OPT_STATIC_ITEM_TILES, args.static_item_tiles)
    scratch = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0")  # 1 GiB cache flush

    r = Runner(m, lib, w, args.which, args)
    res = measure(r, args, scratch, args.steps, args.warmup)
    unions = union_stats(r.idx, w) if args.union_stats and args.which == "forward" and not w.static else None
    fallbacks = None
    if args.which == "forward" and not w.static and args.select_strategy == "fused":
        # one more (untimed) step: how many 64-query selection workgroups
        # walked their candidates twice / took the exact fallback on this data
        m.bsa_select_fallbacks(h, reset=True)
        r.step()
        second, exact = m.bsa_select_fallbacks(h, reset=True)
        fallbacks = {"second_walk": second, "exact_redo": exact,
                     "workgroups": w.batch * w.heads * (-(-w.n // 64))}
    inp, dout_np = r.inp, r.dout_np
    static_mask = None
    if w.static and not args.no_cpu_baseline:
        import oracle
        static_mask = oracle.window_stride_mask(w.n, w.window, w.stride)
    r.close()
    del r
    torch.cuda.empty_cache()

    others = {}
    if not args.only and args.which == "forward":
        for name, ow in W.WORKLOADS.items():
            if name == w.name:
                continue
            print(f"[bench] {name}", file=sys.stderr, flush=True)
            ro = Runner(m, lib, ow, "forward", args)
            o = measure(ro, args, scratch, args.other_steps, 3)
            ro.close()
            del ro
            torch.cuda.empty_cache()
            others[name] = {k: o[k] for k in ("ms_cold_median", "ms_cold_min", "ms_cold_synced_median",
                                              "ms_cold_write_flush_median",
                                              "ms_warm", "tokens_per_s",
                                              "tokens_per_s_warm", "effective_tflops", "algorithmic_gflop",
                                              "page_convention", "stage_ms_per_step", "path_roofline")}
            others[name]["roofline"] = {k: o["roofline"][k] for k in ("kernel", "bound", "achieved", "unit",
                                                                      "frac", "avg_launch_ms")}
            others[name]["config"] = {"batch": ow.batch, "heads": ow.heads, "n": ow.n, "d": ow.d,
                                      "dtype": ow.dtype, "topk": ow.topk, "causal": ow.causal,
                                      "static": ow.static}
    del scratch

    cfg = {"workload": w.name, "batch": w.batch, "heads": w.heads, "n": w.n, "d": w.d, "pass": args.which}
    if w.static:
        cfg.update(window=w.window, stride=w.stride, tile=64, static_item_tiles=args.static_item_tiles or "auto")
    else:
        cfg.update(block=w.block, topk=w.topk, causal=w.causal, select_strategy=args.select_strategy,
                   fine_strategy=args.fine_strategy, panel_chunk_mb=args.panel_chunk_mb or 128,
                   union_rows=args.union_rows,
                   fine_chunk_mb=args.fine_chunk_mb or 1024)
    result = {
        "metric": METRIC if args.which == "forward" else METRIC_BWD,
        "value": res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_cold_median"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": ("synthetic: seeded N(0,1) q/k/v plus per-block key offsets N(0,0.5^2), rounded to bf16 "
                 "(no dataset)") if w.key_offsets else "synthetic: seeded N(0,1) (no dataset)",
        "config": cfg,
        "timing": {"value_from": "median of the cold steps (each queued behind a 1 GiB scratch write and "
                                 "a read of it; HIP events)",
                   "ms_cold_median": res["ms_cold_median"], "ms_cold_min": res["ms_cold_min"],
                   "ms_cold_mean": res["ms_cold_mean"], "ms_warm": res["ms_warm"],
                   "ms_cold_synced_median": res["ms_cold_synced_median"],
                   "ms_cold_write_flush_median": res["ms_cold_write_flush_median"],
                   "tokens_per_s_warm": res["tokens_per_s_warm"]},
        "effective_tflops": res["effective_tflops"],
        "algorithmic_gflop": res["algorithmic_gflop"],
        **({"page_convention": res["page_convention"]} if "page_convention" in res else {}),
        **({"gather_r2": res["gather_r2"]} if "gather_r2" in res else {}),
        "stage_ms_per_step": res["stage_ms_per_step"],
        "roofline": res["roofline"],
        "stage_rooflines": res["stage_rooflines"],
        "path_roofline": res["path_roofline"],
    }
    if others:
        result["workloads"] = others
    if unions:
        result["query_tile_unions"] = unions
    if fallbacks is not None:
        result["select_fallbacks_per_step"] = fallbacks
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = (cpu_baseline(w, inp, args.cpu_positions, static_mask)
                                  if args.which == "forward" else cpu_baseline_backward(w, inp, dout_np))
    lib.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
