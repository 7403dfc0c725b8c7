"""fp64 CPU oracle for the two-stage block-sparse attention forward.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product (the HIP library and its
Python binding) never does.  The arithmetic lives in ``oracle.c`` (plain C,
fp64, OpenMP over rows); this module only compiles it with gcc and marshals
numpy arrays.  It shares no code with the HIP path.

Page references, readings of silent points and the "parity unpinned" list
are in the header of ``oracle.c``; every function here maps 1:1 to one there.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "oracle.c"
_LIB = _HERE / "liboracle.so"
_lib = None


def build(force: bool = True) -> Path:
    """Compile liboracle.so with gcc (IEEE fp64, no fast-math, OpenMP)."""
    if not force and _LIB.exists() and _LIB.stat().st_mtime >= _SRC.stat().st_mtime:
        return _LIB
    tmp = _LIB.with_suffix(".so.tmp")
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off", "-o", str(tmp), str(_SRC), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
        build()
    lib = ctypes.CDLL(str(_LIB))
    P = ctypes.c_void_p
    I = ctypes.c_int64
    lib.oracle_pool.argtypes = [P, I, I, I, I, P]
    lib.oracle_scores.argtypes = [P, P, I, I, I, I, P, I, P]
    lib.oracle_topk.argtypes = [P, P, I, I, I, I, I, ctypes.c_int, P, P, P]
    lib.oracle_attend.argtypes = [P, P, P, I, I, I, I, I, ctypes.c_int, ctypes.c_double, P, P, I, P]
    lib.oracle_window_stride_mask.argtypes = [I, I, I, P]
    lib.oracle_attend_mask.argtypes = [P, P, P, I, I, I, ctypes.c_double, P, P, I, P]
    lib.oracle_visible_pairs.argtypes = [P, P, I, I, I, I, ctypes.c_int]
    lib.oracle_visible_pairs.restype = ctypes.c_int64
    lib.oracle_attend_backward.argtypes = [P, P, P, P, I, I, I, I, I, ctypes.c_int, ctypes.c_double,
                                           P, P, I, P, P, P, I, P, P]
    for name in ("oracle_pool", "oracle_scores", "oracle_topk", "oracle_attend",
                 "oracle_window_stride_mask", "oracle_attend_mask", "oracle_attend_backward"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def set_threads(count: int) -> int:
    """Use `count` OpenMP threads in later calls (the OpenMP runtime the
    library links); returns the count in effect before."""
    lib = _load()
    before = int(lib.omp_get_max_threads())
    lib.omp_set_num_threads(int(count))
    return before


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().omp_get_max_threads())


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a, a.ctypes.data


def _ptr(a):
    return a.ctypes.data


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name} rejected its arguments (rc={rc})")


def _rows(rows, total):
    if rows is None:
        rows = np.arange(total, dtype=np.int64)
    return np.ascontiguousarray(rows, dtype=np.int64)


def _shape(x):
    """[batch, heads, n, d] or [bh, n, d] -> (bh, n, d)."""
    if x.ndim == 4:
        return x.shape[0] * x.shape[1], x.shape[2], x.shape[3]
    if x.ndim == 3:
        return x.shape
    raise ValueError("expected [batch, heads, n, d] or [bh, n, d]")


def pool(k, block):
    """Block representatives, fp64 [bh, nb, d]: the mean of each block's keys."""
    lib = _load()
    bh, n, d = _shape(k)
    k, kp = _f32(k)
    nb = -(-n // block)
    out = np.empty((bh, nb, d), dtype=np.float64)
    _check(lib.oracle_pool(kp, bh, n, d, block, _ptr(out)), "oracle_pool")
    return out


def scores(q, repr_, block, rows=None):
    """Coarse scores q_i . r_beta (unscaled), fp64 [len(rows), nb]."""
    lib = _load()
    bh, n, d = _shape(q)
    q, qp = _f32(q)
    repr_ = np.ascontiguousarray(repr_, dtype=np.float64)
    nb = -(-n // block)
    assert repr_.shape == (bh, nb, d)
    rows = _rows(rows, bh * n)
    out = np.empty((rows.size, nb), dtype=np.float64)
    _check(lib.oracle_scores(qp, _ptr(repr_), bh, n, d, block, _ptr(rows), rows.size,
                             _ptr(out)), "oracle_scores")
    return out


def topk(scores_, n, block, k, causal, rows=None):
    """Per-row top-k block selection.

    Returns (idx int32 [rows, k] ascending, -1 padded; kth; next) where kth and
    next are the k_eff-th and (k_eff+1)-th candidate scores (NaN if absent)."""
    lib = _load()
    scores_ = np.ascontiguousarray(scores_, dtype=np.float64)
    nrows, nb = scores_.shape
    rows = _rows(rows, nrows)
    assert rows.size == nrows
    idx = np.empty((nrows, k), dtype=np.int32)
    kth = np.empty(nrows, dtype=np.float64)
    nxt = np.empty(nrows, dtype=np.float64)
    _check(lib.oracle_topk(_ptr(scores_), _ptr(rows), nrows, n, nb, block, k, int(causal),
                           _ptr(idx), _ptr(kth), _ptr(nxt)), "oracle_topk")
    return idx, kth, nxt


def attend(q, k, v, idx, block, causal, scale, rows=None):
    """Fine attention over the selected blocks, fp64 [rows, d]."""
    lib = _load()
    bh, n, d = _shape(q)
    q, qp = _f32(q)
    k, kp = _f32(k)
    v, vp = _f32(v)
    rows = _rows(rows, bh * n)
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(rows.size, -1)
    out = np.empty((rows.size, d), dtype=np.float64)
    _check(lib.oracle_attend(qp, kp, vp, bh, n, d, block, idx.shape[1], int(causal),
                             float(scale), _ptr(idx), _ptr(rows), rows.size, _ptr(out)),
           "oracle_attend")
    return out


def select(q, k, block, topk_, causal, rows=None):
    """Stage 1 end to end: pool, score, select.  Returns (idx, kth, next)."""
    bh, n, d = _shape(q)
    r = pool(k, block)
    s = scores(q, r, block, rows)
    rows = _rows(rows, bh * n)
    return topk(s, n, block, topk_, causal, rows)


def forward(q, k, v, block, topk_, causal, scale, rows=None):
    """Both stages.  Returns (out fp64 [rows, d], idx, kth, next)."""
    bh, n, d = _shape(q)
    rows = _rows(rows, bh * n)
    idx, kth, nxt = select(q, k, block, topk_, causal, rows)
    out = attend(q, k, v, idx, block, causal, scale, rows)
    return out, idx, kth, nxt


def window_stride_mask(n, window, stride):
    """uint8 [n, n]: 1 where |i - j| <= window or j % stride == 0."""
    lib = _load()
    m = np.empty((n, n), dtype=np.uint8)
    _check(lib.oracle_window_stride_mask(n, window, stride, _ptr(m)), "oracle_window_stride_mask")
    return m


def attend_backward(q, k, v, dout, idx, block, causal, scale, rows=None, key_blocks=None):
    """Gradients of the fine attention with the selection idx held fixed.

    idx: int32 selections of ALL bh*n rows ([bh*n, topk], -1 padded).
    rows: query rows for dq and lse (default all); key_blocks: flattened
    (head * nb + beta) ids for dk and dv (default all).
    Returns (dq [rows, d], lse [rows], dk [blocks, block, d], dv [same]), fp64."""
    lib = _load()
    bh, n, d = _shape(q)
    nb = -(-n // block)
    q, qp = _f32(q)
    k, kp = _f32(k)
    v, vp = _f32(v)
    dout, dp = _f32(dout)
    rows = _rows(rows, bh * n)
    kb = np.arange(bh * nb, dtype=np.int64) if key_blocks is None else \
        np.ascontiguousarray(key_blocks, dtype=np.int64)
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(bh * n, -1)
    dq = np.empty((rows.size, d), dtype=np.float64)
    lse = np.empty(rows.size, dtype=np.float64)
    dk = np.empty((kb.size, block, d), dtype=np.float64)
    dv = np.empty((kb.size, block, d), dtype=np.float64)
    _check(lib.oracle_attend_backward(qp, kp, vp, dp, bh, n, d, block, idx.shape[1], int(causal),
                                      float(scale), _ptr(idx), _ptr(rows), rows.size, _ptr(dq),
                                      _ptr(lse), _ptr(kb), kb.size, _ptr(dk), _ptr(dv)),
           "oracle_attend_backward")
    return dq, lse, dk, dv


def attend_mask(q, k, v, mask, scale, rows=None):
    """Softmax attention under an explicit [n, n] key mask, fp64 [rows, d]."""
    lib = _load()
    bh, n, d = _shape(q)
    q, qp = _f32(q)
    k, kp = _f32(k)
    v, vp = _f32(v)
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    assert mask.shape == (n, n)
    rows = _rows(rows, bh * n)
    out = np.empty((rows.size, d), dtype=np.float64)
    _check(lib.oracle_attend_mask(qp, kp, vp, bh, n, d, float(scale), _ptr(mask), _ptr(rows),
                                  rows.size, _ptr(out)), "oracle_attend_mask")
    return out


def visible_pairs(idx, n, block, causal, rows):
    """Number of (query, key) pairs the fine stage visits."""
    lib = _load()
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(rows.size, -1)
    return int(lib.oracle_visible_pairs(_ptr(idx), _ptr(rows), rows.size, n, block,
                                        idx.shape[1], int(causal)))
