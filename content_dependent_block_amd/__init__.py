"""Two-stage, content-dependent block-sparse attention forward for AMD MI355X.

Stage 1 mean-pools each 64-key block, scores every query against every block
representative and keeps each query's top-k blocks; stage 2 runs fused
online-softmax attention over only those blocks.  ``block_sparse_attention``
is the differentiable form (the selection is held fixed in the backward).  All
of it runs in the gfx950 kernels of ``libbsa.so`` behind the C ABI in
``include/bsa.h``; this package is a thin binding with the same names (see
``_binding``).
"""
from __future__ import annotations

import math

import torch

from ._binding import *  # noqa: F401,F403  (bsa_* functions and constants)
from ._binding import (EXPORTED, STAGE_NAMES, BsaError, bsa_backward, bsa_backward_varlen, bsa_create,
                       bsa_destroy, bsa_forward, bsa_forward_budgets, bsa_forward_static, bsa_forward_train,
                       bsa_forward_varlen, bsa_tiles_create)


class BlockSparseAttention:
    """Owns a library handle (and its workspace) on one device."""

    def __init__(self, device: int = 0):
        self.device = device
        self.handle = bsa_create(device)

    def close(self):
        if self.handle is not None:
            bsa_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def forward(self, q, k, v, *, topk, block: int = 64, scale: float | None = None,
                causal: bool = False, return_indices: bool = False, stream=None):
        """out (float32, same shape as q), and optionally the int32 block indices.

        topk: one budget for every head, or a sequence with one per head (the
        index rows then have max(topk) entries, -1 padded)."""
        b, h, n, d = q.shape
        scale = 1.0 / math.sqrt(d) if scale is None else scale
        per_head = not isinstance(topk, int)
        kmax = int(max(topk)) if per_head else topk
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        idx = torch.empty((b, h, n, kmax), dtype=torch.int32, device=q.device) if return_indices else None
        if per_head:
            bsa_forward_budgets(self.handle, q, k, v, out, idx, head_topk=list(topk), topk_max=kmax,
                                block=block, scale=scale, causal=causal, stream=stream)
        else:
            bsa_forward(self.handle, q, k, v, out, idx, block=block, topk=topk, scale=scale,
                        causal=causal, stream=stream)
        return (out, idx) if return_indices else out

    def forward_varlen(self, q, k, v, cu_seqlens, *, topk, block: int = 64, scale: float | None = None,
                       causal: bool = False, return_indices: bool = False, stream=None):
        """A batch of sequences of different lengths: q, k, v [heads, total, d],
        sequence i = rows cu_seqlens[i] .. cu_seqlens[i+1]-1 of every head,
        each attended to on its own.  out float32 [heads, total, d], and
        optionally the int32 indices [heads, total, max(topk)], numbered from
        each sequence's first block.  topk: an int or one per head."""
        h, total, d = q.shape
        scale = 1.0 / math.sqrt(d) if scale is None else scale
        per_head = not isinstance(topk, int)
        kmax = int(max(topk)) if per_head else int(topk)
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        idx = torch.empty((h, total, kmax), dtype=torch.int32, device=q.device) if return_indices else None
        bsa_forward_varlen(self.handle, q, k, v, out, cu_seqlens, idx, topk=kmax,
                           head_topk=list(topk) if per_head else None, block=block, scale=scale,
                           causal=causal, stream=stream)
        return (out, idx) if return_indices else out

    def tiles(self, n: int, row_ptr, col, rowmask=None):
        """A device tile list (validated on the host) for forward_static."""
        return bsa_tiles_create(self.handle, n, row_ptr, col, rowmask)

    def forward_static(self, q, k, v, tiles, *, scale: float | None = None, stream=None):
        d = q.shape[-1]
        scale = 1.0 / math.sqrt(d) if scale is None else scale
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        bsa_forward_static(self.handle, q, k, v, out, tiles, scale=scale, stream=stream)
        return out


class _BlockSparseAttentionFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, lib, topk, head_topk, block, scale, causal, cu_seqlens):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        idx = torch.empty((*q.shape[:-1], topk), dtype=torch.int32, device=q.device)
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
        if cu_seqlens is None:
            bsa_forward_train(lib.handle, q, k, v, out, idx, lse, topk=topk, head_topk=head_topk,
                              block=block, scale=scale, causal=causal)
        else:
            bsa_forward_varlen(lib.handle, q, k, v, out, cu_seqlens, idx, lse, topk=topk, head_topk=head_topk,
                               block=block, scale=scale, causal=causal)
        ctx.save_for_backward(q, k, v, out, idx, lse)
        ctx.lib, ctx.block, ctx.scale, ctx.causal = lib, block, scale, causal
        ctx.cu_seqlens = cu_seqlens
        ctx.mark_non_differentiable(idx)
        return out, idx

    @staticmethod
    def backward(ctx, dout, _didx):
        q, k, v, out, idx, lse = ctx.saved_tensors
        dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        dk = torch.empty_like(dq)
        dv = torch.empty_like(dq)
        if ctx.cu_seqlens is None:
            bsa_backward(ctx.lib.handle, q, k, v, out, dout.contiguous().float(), idx, lse, dq, dk, dv,
                         block=ctx.block, scale=ctx.scale, causal=ctx.causal)
        else:
            bsa_backward_varlen(ctx.lib.handle, q, k, v, out, dout.contiguous().float(), idx, lse, dq, dk, dv,
                                ctx.cu_seqlens, block=ctx.block, scale=ctx.scale, causal=ctx.causal)
        return dq, dk, dv, None, None, None, None, None, None, None


def block_sparse_attention(q, k, v, topk, *, lib: BlockSparseAttention, block: int = 64,
                           scale: float | None = None, causal: bool = False,
                           return_indices: bool = False, cu_seqlens=None):
    """Differentiable two-stage block-sparse attention: float32 out (and the
    int32 selection).  topk: an int, or one int per head (rows then hold
    max(topk) indices, -1 padded).  q, k, v: [batch, heads, n, d], or with
    cu_seqlens (nseq + 1 ints) a batch of sequences of different lengths,
    [heads, total, d].  Gradients reach q, k, v through the fine stage; the
    selection is a discrete choice and is held fixed."""
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    per_head = not isinstance(topk, int)
    kmax = int(max(topk)) if per_head else int(topk)
    cu = None if cu_seqlens is None else [int(x) for x in cu_seqlens]
    out, idx = _BlockSparseAttentionFn.apply(q, k, v, lib, kmax, list(topk) if per_head else None,
                                             block, scale, causal, cu)
    return (out, idx) if return_indices else out
