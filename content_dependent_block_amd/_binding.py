"""ctypes binding of libbsa.so (include/bsa.h), same names as the C ABI.

Argument marshalling only: tensors are checked for shape, dtype, device and
contiguity (the C side cannot see sizes), then their device pointers and the
current HIP stream are passed through.  Every step of the computation runs in
the gfx950 kernels of libbsa.so; there is no fallback.  If the library has not
been built, importing this module raises ImportError.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

import numpy as np
import torch

_LIB_PATH = Path(__file__).resolve().parent / "libbsa.so"
if not _LIB_PATH.exists():
    raise ImportError(f"{_LIB_PATH} is not built; run `python -m content_dependent_block_amd.build`")
_lib = ctypes.CDLL(str(_LIB_PATH))

BSA_OK, BSA_ERR_INVALID_ARG, BSA_ERR_UNSUPPORTED = 0, 1, 2
BSA_ERR_NO_DEVICE, BSA_ERR_OUT_OF_MEMORY, BSA_ERR_LAUNCH = 3, 4, 5
BSA_FP32, BSA_BF16 = 0, 1
BSA_STAGE_POOL, BSA_STAGE_COARSE, BSA_STAGE_TOPK, BSA_STAGE_FINE = 0, 1, 2, 3
BSA_STAGE_GATHER_INDEX, BSA_STAGE_GATHER_COMBINE, BSA_STAGE_COARSE_TOPK = 4, 5, 6
BSA_STAGE_BWD_PREP, BSA_STAGE_BWD_INDEX, BSA_STAGE_BWD_PAIRS, BSA_STAGE_BWD_REDUCE = 7, 8, 9, 10
BSA_STAGE_RAGGED_COPY = 11
BSA_STAGE_STATIC_COMBINE = 12
BSA_NUM_STAGES = 13
STAGE_NAMES = ("block_pool", "coarse_score", "topk_select", "sparse_flash_fwd", "gather_index",
               "gather_combine", "coarse_select", "bwd_prep", "bwd_index", "bwd_pairs", "bwd_reduce",
               "ragged_copy", "static_combine")
BSA_OPT_PANEL_CHUNK_BYTES, BSA_OPT_FINE_STRATEGY, BSA_OPT_FINE_CHUNK_BYTES = 0, 1, 2
BSA_OPT_SELECT_STRATEGY = 3
BSA_OPT_STATIC_ITEM_TILES = 4
BSA_OPT_UNION_ROWS = 5
BSA_FINE_BLOCK_GATHER, BSA_FINE_QUERY_TILE, BSA_FINE_PER_QUERY = 0, 1, 2
BSA_SELECT_FUSED, BSA_SELECT_PANEL = 0, 1

_P, _I, _I64, _F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float


def _sig(name, args, res=ctypes.c_int):
    f = getattr(_lib, name)
    f.argtypes, f.restype = args, res
    return f


_sig("bsa_create", [_I, ctypes.POINTER(_P)])
_sig("bsa_destroy", [_P])
_sig("bsa_status_string", [_I], ctypes.c_char_p)
_sig("bsa_last_error", [_P], ctypes.c_char_p)
_sig("bsa_set_option", [_P, _I, _I64])
_sig("bsa_workspace_bytes", [_P, ctypes.POINTER(ctypes.c_size_t)])
_sig("bsa_forward", [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P])
_sig("bsa_forward_noalloc", [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P])
_sig("bsa_forward_budgets", [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _I, _F, _I, _P])
_sig("bsa_forward_train", [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _I, _F, _I, _P])
_sig("bsa_backward", [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I,
                      _P])
_sig("bsa_forward_varlen", [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _I, _F, _I, _P])
_sig("bsa_backward_varlen", [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I,
                             _P])
_sig("bsa_fine_forward", [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P])
_sig("bsa_block_pool", [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P])
_sig("bsa_coarse_score", [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P])
_sig("bsa_topk_select", [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P])
_sig("bsa_tiles_create", [_P, _I, _I, _P, _P, _P, _I64, ctypes.POINTER(_P)])
_sig("bsa_tiles_destroy", [_P])
_sig("bsa_forward_static", [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _F, _P])
_sig("bsa_tiles_from_mask", [_P, _I, _I, _P, _P, _P, ctypes.POINTER(_I64)])
_sig("bsa_tiles_window_stride", [_I, _I, _I, _I, _P, _P, _P, ctypes.POINTER(_I64)])
_sig("bsa_tiles_validate", [_P, _P, _I64, _I, _I])
_sig("bsa_profile_enable", [_P, _I])
_sig("bsa_profile_read", [_P, _P, _P, _I])
_sig("bsa_select_fallbacks", [_P, _P, _I])

EXPORTED = ("bsa_create", "bsa_destroy", "bsa_status_string", "bsa_last_error", "bsa_set_option",
            "bsa_workspace_bytes", "bsa_forward", "bsa_forward_noalloc", "bsa_forward_budgets",
            "bsa_forward_train",
            "bsa_backward", "bsa_forward_varlen", "bsa_backward_varlen", "bsa_fine_forward",
            "bsa_block_pool",
            "bsa_coarse_score", "bsa_topk_select", "bsa_tiles_create", "bsa_tiles_destroy",
            "bsa_forward_static", "bsa_tiles_from_mask",
            "bsa_tiles_window_stride", "bsa_tiles_validate", "bsa_profile_enable",
            "bsa_profile_read", "bsa_select_fallbacks")


class BsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{bsa_status_string(status)}: {message}")
        self.status = status


def bsa_status_string(status: int) -> str:
    return _lib.bsa_status_string(status).decode()


def bsa_last_error(h=None) -> str:
    return _lib.bsa_last_error(h).decode()


def _check(status: int, h=None):
    if status != BSA_OK:
        raise BsaError(status, bsa_last_error(h))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BSA_BF16
    if t.dtype == torch.float32:
        return BSA_FP32
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


# The current stream's raw handle without building a Stream object (about a
# microsecond and a half less per call), where this torch has the accessor.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, device):
    if stream is None:
        if _raw_stream is not None:
            return ctypes.c_void_p(_raw_stream(device.index if device.index is not None
                                               else torch.cuda.current_device()))
        return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _need(t, name, shape, dtype, device):
    # the common case in one test; anything else takes the checks below,
    # which name what is wrong
    if (isinstance(t, torch.Tensor) and t.shape == shape and (dtype is None or t.dtype == dtype)
            and t.device == device and t.is_contiguous()):
        return ctypes.c_void_p(t.data_ptr())
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _qkv(q, k, v):
    if q.dim() != 4:
        raise ValueError("q must be [batch, heads, n, d]")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    if (isinstance(k, torch.Tensor) and isinstance(v, torch.Tensor) and k.dtype is q.dtype and v.dtype is q.dtype
            and k.shape == q.shape and v.shape == q.shape and k.device == dev and v.device == dev
            and q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        return ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()), dev
    pq = _need(q, "q", q.shape, None, dev)
    pk = _need(k, "k", q.shape, q.dtype, dev)
    pv = _need(v, "v", q.shape, q.dtype, dev)
    return pq, pk, pv, dev


# ------------------------------------------------------------- lifetime --
def bsa_create(device: int = 0):
    h = ctypes.c_void_p()
    _check(_lib.bsa_create(device, ctypes.byref(h)))
    return h


def bsa_destroy(h) -> None:
    _check(_lib.bsa_destroy(h), h)


def bsa_set_option(h, option: int, value: int) -> None:
    _check(_lib.bsa_set_option(h, option, value), h)


def bsa_workspace_bytes(h) -> int:
    out = ctypes.c_size_t()
    _check(_lib.bsa_workspace_bytes(h, ctypes.byref(out)), h)
    return int(out.value)


# -------------------------------------------------------------- forward --
def bsa_forward(h, q, k, v, out, block_idx_out=None, *, block: int = 64, topk: int,
                scale: float, causal: bool = False, stream=None) -> None:
    pq, pk, pv, dev = _qkv(q, k, v)
    b, hh, n, d = q.shape
    po = _need(out, "out", q.shape, torch.float32, dev)
    pi = None
    if block_idx_out is not None:
        pi = _need(block_idx_out, "block_idx_out", (b, hh, n, topk), torch.int32, dev)
    _check(_lib.bsa_forward(h, pq, pk, pv, po, pi, b, hh, n, d, _dtype_code(q), block, topk,
                            float(scale), int(causal), _stream(stream, dev)), h)


def bsa_forward_noalloc(h, q, k, v, out, block_idx_out, *, block: int = 64, topk: int,
                        scale: float, causal: bool = False, stream=None) -> None:
    """bsa_forward with no device allocation: the workspace is the library's
    fixed per-device array (calls that overlap on one device race)."""
    pq, pk, pv, dev = _qkv(q, k, v)
    b, hh, n, d = q.shape
    po = _need(out, "out", q.shape, torch.float32, dev)
    pi = _need(block_idx_out, "block_idx_out", (b, hh, n, topk), torch.int32, dev)
    _check(_lib.bsa_forward_noalloc(h, pq, pk, pv, po, pi, b, hh, n, d, _dtype_code(q), block, topk,
                                    float(scale), int(causal), _stream(stream, dev)), h)


def bsa_forward_budgets(h, q, k, v, out, block_idx_out=None, *, head_topk, topk_max: int = None,
                        block: int = 64, scale: float, causal: bool = False, stream=None) -> None:
    """bsa_forward with one top-k budget per head (head_topk: ints, one per head)."""
    pq, pk, pv, dev = _qkv(q, k, v)
    b, hh, n, d = q.shape
    ks = np.ascontiguousarray(np.asarray(head_topk, dtype=np.int32).reshape(-1))
    if ks.size != hh:
        raise ValueError(f"head_topk needs {hh} entries, got {ks.size}")
    if topk_max is None:
        topk_max = int(ks.max())
    po = _need(out, "out", q.shape, torch.float32, dev)
    pi = None
    if block_idx_out is not None:
        pi = _need(block_idx_out, "block_idx_out", (b, hh, n, topk_max), torch.int32, dev)
    _check(_lib.bsa_forward_budgets(h, pq, pk, pv, po, pi, b, hh, n, d, _dtype_code(q), block,
                                    ks.ctypes.data, int(topk_max), float(scale), int(causal),
                                    _stream(stream, dev)), h)


def bsa_forward_train(h, q, k, v, out, block_idx_out, lse_out, *, topk: int, head_topk=None,
                      block: int = 64, scale: float, causal: bool = False, stream=None) -> None:
    """bsa_forward that also writes the row log-sum-exp the backward needs;
    head_topk (optional, one int per head) as in bsa_forward_budgets."""
    pq, pk, pv, dev = _qkv(q, k, v)
    b, hh, n, d = q.shape
    po = _need(out, "out", q.shape, torch.float32, dev)
    pi = _need(block_idx_out, "block_idx_out", (b, hh, n, topk), torch.int32, dev)
    pl = _need(lse_out, "lse_out", (b, hh, n), torch.float32, dev)
    pk_ = None
    if head_topk is not None:
        ks = np.ascontiguousarray(np.asarray(head_topk, dtype=np.int32).reshape(-1))
        if ks.size != hh:
            raise ValueError(f"head_topk needs {hh} entries, got {ks.size}")
        pk_ = ks.ctypes.data
    _check(_lib.bsa_forward_train(h, pq, pk, pv, po, pi, pl, b, hh, n, d, _dtype_code(q), block, pk_,
                                  int(topk), float(scale), int(causal), _stream(stream, dev)), h)


def bsa_backward(h, q, k, v, out, dout, block_idx, lse, dq, dk, dv, *, block: int = 64,
                 scale: float, causal: bool = False, stream=None) -> None:
    """Gradients of q, k, v through the fine stage (selection fixed)."""
    pq, pk, pv, dev = _qkv(q, k, v)
    b, hh, n, d = q.shape
    if block_idx.dim() != 4:
        raise ValueError("block_idx must be [batch, heads, n, topk]")
    topk = block_idx.shape[-1]
    f32 = torch.float32
    args = [_need(out, "out", q.shape, f32, dev), _need(dout, "dout", q.shape, f32, dev),
            _need(block_idx, "block_idx", (b, hh, n, topk), torch.int32, dev),
            _need(lse, "lse", (b, hh, n), f32, dev), _need(dq, "dq", q.shape, f32, dev),
            _need(dk, "dk", q.shape, f32, dev), _need(dv, "dv", q.shape, f32, dev)]
    _check(_lib.bsa_backward(h, pq, pk, pv, *args, b, hh, n, d, _dtype_code(q), block, topk,
                             float(scale), int(causal), _stream(stream, dev)), h)


def _cu_seqlens(cu_seqlens):
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32).reshape(-1))
    if cu.size < 2:
        raise ValueError("cu_seqlens needs nseq + 1 >= 2 entries")
    return cu, cu.size - 1, int(cu[-1])


def _qkv_varlen(q, k, v, total):
    if q.dim() != 3:
        raise ValueError("q must be [heads, total, d] for a variable-length batch")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    if q.shape[1] != total:
        raise ValueError(f"q has {q.shape[1]} rows per head, cu_seqlens ends at {total}")
    pq = _need(q, "q", q.shape, None, dev)
    pk = _need(k, "k", q.shape, q.dtype, dev)
    pv = _need(v, "v", q.shape, q.dtype, dev)
    return pq, pk, pv, dev


def bsa_forward_varlen(h, q, k, v, out, cu_seqlens, block_idx_out=None, lse_out=None, *, topk: int,
                       head_topk=None, block: int = 64, scale: float, causal: bool = False,
                       stream=None) -> None:
    """Both stages over a batch of sequences of different lengths: q, k, v
    [heads, total, d], sequence i = rows cu_seqlens[i] .. cu_seqlens[i+1]-1 of
    every head; block_idx_out [heads, total, topk] (block numbers from each
    sequence's first block), lse_out [heads, total] (both optional)."""
    cu, nseq, total = _cu_seqlens(cu_seqlens)
    pq, pk, pv, dev = _qkv_varlen(q, k, v, total)
    hh, _, d = q.shape
    po = _need(out, "out", q.shape, torch.float32, dev)
    pi = None if block_idx_out is None else _need(block_idx_out, "block_idx_out", (hh, total, topk),
                                                  torch.int32, dev)
    pl = None if lse_out is None else _need(lse_out, "lse_out", (hh, total), torch.float32, dev)
    pk_ = None
    if head_topk is not None:
        ks = np.ascontiguousarray(np.asarray(head_topk, dtype=np.int32).reshape(-1))
        if ks.size != hh:
            raise ValueError(f"head_topk needs {hh} entries, got {ks.size}")
        pk_ = ks.ctypes.data
    _check(_lib.bsa_forward_varlen(h, pq, pk, pv, po, pi, pl, cu.ctypes.data, nseq, hh, d, _dtype_code(q),
                                   block, pk_, int(topk), float(scale), int(causal), _stream(stream, dev)), h)


def bsa_backward_varlen(h, q, k, v, out, dout, block_idx, lse, dq, dk, dv, cu_seqlens, *, block: int = 64,
                        scale: float, causal: bool = False, stream=None) -> None:
    """Gradients of q, k, v for a batch laid out as for bsa_forward_varlen."""
    cu, nseq, total = _cu_seqlens(cu_seqlens)
    pq, pk, pv, dev = _qkv_varlen(q, k, v, total)
    hh, _, d = q.shape
    if block_idx.dim() != 3:
        raise ValueError("block_idx must be [heads, total, topk]")
    topk = block_idx.shape[-1]
    f32 = torch.float32
    args = [_need(out, "out", q.shape, f32, dev), _need(dout, "dout", q.shape, f32, dev),
            _need(block_idx, "block_idx", (hh, total, topk), torch.int32, dev),
            _need(lse, "lse", (hh, total), f32, dev), _need(dq, "dq", q.shape, f32, dev),
            _need(dk, "dk", q.shape, f32, dev), _need(dv, "dv", q.shape, f32, dev)]
    _check(_lib.bsa_backward_varlen(h, pq, pk, pv, *args, cu.ctypes.data, nseq, hh, d, _dtype_code(q), block,
                                    topk, float(scale), int(causal), _stream(stream, dev)), h)


def bsa_fine_forward(h, q, k, v, out, block_idx, *, block: int = 64, scale: float,
                     causal: bool = False, stream=None) -> None:
    pq, pk, pv, dev = _qkv(q, k, v)
    b, hh, n, d = q.shape
    if block_idx.dim() != 4:
        raise ValueError("block_idx must be [batch, heads, n, topk]")
    topk = block_idx.shape[-1]
    po = _need(out, "out", q.shape, torch.float32, dev)
    pi = _need(block_idx, "block_idx", (b, hh, n, topk), torch.int32, dev)
    _check(_lib.bsa_fine_forward(h, pq, pk, pv, po, pi, b, hh, n, d, _dtype_code(q), block, topk,
                                 float(scale), int(causal), _stream(stream, dev)), h)


def bsa_block_pool(h, k, repr_out, *, block: int = 64, stream=None) -> None:
    if k.dim() != 4:
        raise ValueError("k must be [batch, heads, n, d]")
    b, hh, n, d = k.shape
    dev = k.device
    pk = _need(k, "k", k.shape, None, dev)
    pr = _need(repr_out, "repr_out", (b, hh, n // block, d), torch.float32, dev)
    _check(_lib.bsa_block_pool(h, pk, pr, b, hh, n, d, _dtype_code(k), block, _stream(stream, dev)), h)


def bsa_coarse_score(h, q, repr_, panel_out, *, block: int = 64, causal: bool = False,
                     stream=None) -> None:
    if q.dim() != 4:
        raise ValueError("q must be [batch, heads, n, d]")
    b, hh, n, d = q.shape
    dev = q.device
    pq = _need(q, "q", q.shape, None, dev)
    pr = _need(repr_, "repr", (b, hh, n // block, d), torch.float32, dev)
    pp = _need(panel_out, "panel_out", (n // block, b * hh * n), torch.float32, dev)
    _check(_lib.bsa_coarse_score(h, pq, pr, pp, b, hh, n, d, _dtype_code(q), block, int(causal),
                                 _stream(stream, dev)), h)


def bsa_topk_select(h, panel, block_idx_out, *, block: int = 64, causal: bool = False,
                    stream=None) -> None:
    """panel: block-major [n/block, batch*heads*n] as bsa_coarse_score writes it;
    block_idx_out: [batch, heads, n, topk]."""
    if block_idx_out.dim() != 4:
        raise ValueError("block_idx_out must be [batch, heads, n, topk]")
    b, hh, n, topk = block_idx_out.shape
    dev = panel.device
    pp = _need(panel, "panel", (n // block, b * hh * n), torch.float32, dev)
    pi = _need(block_idx_out, "block_idx_out", (b, hh, n, topk), torch.int32, dev)
    _check(_lib.bsa_topk_select(h, pp, pi, b, hh, n, block, topk, int(causal),
                                _stream(stream, dev)), h)


# --------------------------------------------------------------- static --
class TileList:
    """A validated tile list in device memory (bsa_tiles_create); free it with
    close() or use it as a context manager."""

    def __init__(self, h, n: int, row_ptr, col, rowmask=None, tile: int = 64):
        row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
        col = np.ascontiguousarray(col, dtype=np.int32)
        if row_ptr.size != -(-n // tile) + 1:
            raise ValueError(f"row_ptr needs {-(-n // tile) + 1} entries, got {row_ptr.size}")
        pm = None
        if rowmask is not None:
            rowmask = np.ascontiguousarray(rowmask).view(np.uint64).reshape(-1, tile)
            if rowmask.shape[0] != col.size:
                raise ValueError(f"rowmask needs {col.size} rows of {tile}, got {rowmask.shape[0]}")
            pm = rowmask.ctypes.data
        self.n, self.nnz = n, int(col.size)
        self.ptr = ctypes.c_void_p()
        _check(_lib.bsa_tiles_create(h, n, tile, row_ptr.ctypes.data, col.ctypes.data if col.size else None,
                                     pm, col.size, ctypes.byref(self.ptr)), h)

    def close(self) -> None:
        if self.ptr:
            _check(_lib.bsa_tiles_destroy(self.ptr))
            self.ptr = ctypes.c_void_p()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def bsa_tiles_create(h, n: int, row_ptr, col, rowmask=None, tile: int = 64) -> TileList:
    """Validate a host tile list and copy it to the device (a TileList)."""
    return TileList(h, n, row_ptr, col, rowmask, tile)


def bsa_tiles_destroy(tiles: TileList) -> None:
    tiles.close()


def bsa_forward_static(h, q, k, v, out, tiles: TileList, *, scale: float, tile: int = 64,
                       stream=None) -> None:
    pq, pk, pv, dev = _qkv(q, k, v)
    b, hh, n, d = q.shape
    po = _need(out, "out", q.shape, torch.float32, dev)
    _check(_lib.bsa_forward_static(h, pq, pk, pv, po, b, hh, n, d, _dtype_code(q), tile, tiles.ptr,
                                   float(scale), _stream(stream, dev)), h)


def _tiles(fn, n, *head_args):
    row_ptr = np.zeros(-(-n // 64) + 1, dtype=np.int32)
    nnz = ctypes.c_int64(0)
    _check(fn(*head_args, row_ptr.ctypes.data, None, None, ctypes.byref(nnz)))
    col = np.zeros(max(nnz.value, 1), dtype=np.int32)
    rowmask = np.zeros((max(nnz.value, 1), 64), dtype=np.uint64)
    _check(fn(*head_args, row_ptr.ctypes.data, col.ctypes.data, rowmask.ctypes.data,
              ctypes.byref(nnz)))
    return row_ptr, col[: nnz.value].copy(), rowmask[: nnz.value].copy()


def bsa_tiles_from_mask(mask: np.ndarray, tile: int = 64):
    """Host CSR tile list (row_ptr, col, rowmask) of a dense [n, n] mask."""
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    n = mask.shape[0]
    if mask.shape != (n, n):
        raise ValueError("mask must be square")
    return _tiles(_lib.bsa_tiles_from_mask, n, mask.ctypes.data, n, tile)


def bsa_tiles_window_stride(n: int, window: int, stride: int, tile: int = 64):
    """Host CSR tile list of the window+stride pattern."""
    return _tiles(_lib.bsa_tiles_window_stride, n, n, window, stride, tile)


def bsa_tiles_validate(row_ptr: np.ndarray, col: np.ndarray, n: int, tile: int = 64) -> bool:
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
    col = np.ascontiguousarray(col, dtype=np.int32)
    if row_ptr.size != -(-n // tile) + 1:
        return False
    return _lib.bsa_tiles_validate(row_ptr.ctypes.data, col.ctypes.data if col.size else None,
                                   col.size, n, tile) == BSA_OK


# --------------------------------------------------------------- timing --
def bsa_profile_enable(h, on: bool = True) -> None:
    _check(_lib.bsa_profile_enable(h, int(on)), h)


def bsa_profile_read(h, reset: bool = True):
    """Per-stage summed kernel milliseconds and launch counts."""
    ms = (ctypes.c_double * BSA_NUM_STAGES)()
    launches = (ctypes.c_int64 * BSA_NUM_STAGES)()
    _check(_lib.bsa_profile_read(h, ms, launches, int(reset)), h)
    return list(ms), list(launches)


def bsa_select_fallbacks(h, reset: bool = False):
    """(second walks, exact redos): fused-selection workgroups that walked
    their candidates a second time / took the exact fallback on this handle
    (waits for the device)."""
    c = (ctypes.c_int64 * 2)()
    _check(_lib.bsa_select_fallbacks(h, c, int(reset)), h)
    return int(c[0]), int(c[1])
