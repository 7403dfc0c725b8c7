"""bsa_forward_noalloc (the entry point for callers that cannot allocate)
against bsa_forward, through the C ABI, on two calls in a row, the second
with a smaller input.  Marked gpu."""
import ctypes
import sys

import numpy as np
import pytest

import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(inp, dtype):
    if dtype == "bf16":
        conv = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
        return conv(inp.q_bits), conv(inp.k_bits), conv(inp.v_bits)
    return tuple(torch.from_numpy(x).cuda() for x in (inp.q, inp.k, inp.v))


def call(L, h, fn, w, qkv, topk, causal):
    q, k, v = qkv
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full(q.shape[:3] + (topk,), -7, dtype=torch.int32, device="cuda")
    st = getattr(L, fn)(h, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), idx.data_ptr(),
                        q.shape[0], q.shape[1], q.shape[2], q.shape[3], 1 if w.dtype == "bf16" else 0, 64,
                        topk, ctypes.c_float(w.scale), int(causal), None)
    assert st == 0, f"{fn} returned {st}"
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy()


@pytest.mark.parametrize("first,second", [
    (("dyn_bf16_n32k", 8, 32768, 16, False), ("dyn_bf16_n4k", 8, 4096, 16, False)),
    (("causal_bf16_n128k", 2, 16384, 32, True), ("tiny_fp32_n1k", 1, 1024, 4, True)),
])
def test_noalloc_matches_bsa_forward(first, second):
    """Each call's indices and outputs equal bsa_forward's bit for bit (the
    same kernels; the fine stage's row chunks differ, which changes no
    result); the second, smaller call runs on the array the first left."""
    import content_dependent_block_amd as m
    L = m._binding._lib
    with m.BlockSparseAttention(0) as lib:
        for name, heads, n, topk, causal in (first, second):
            w = W.WORKLOADS[name]
            inp = W.generate(w, n=n, heads=heads)
            qkv = to_dev(inp, w.dtype)
            say(f"[gpu] bsa_forward_noalloc {name} heads={heads} n={n} k={topk} causal={causal}")
            o_ref, i_ref = call(L, lib.handle, "bsa_forward", w, qkv, topk, causal)
            o, i = call(L, lib.handle, "bsa_forward_noalloc", w, qkv, topk, causal)
            assert np.array_equal(i, i_ref)
            assert np.array_equal(o.view(np.uint32), o_ref.view(np.uint32))


def test_noalloc_refuses_what_does_not_fit():
    """A problem whose representatives exceed the fixed array is refused with
    BSA_ERR_UNSUPPORTED before anything is enqueued; ragged n likewise."""
    import content_dependent_block_amd as m
    L = m._binding._lib
    with m.BlockSparseAttention(0) as lib:
        q = torch.zeros((1, 1, 128, 64), dtype=torch.bfloat16, device="cuda")
        out = torch.zeros((1, 1, 128, 64), dtype=torch.float32, device="cuda")
        idx = torch.zeros((1, 1, 128, 4), dtype=torch.int32, device="cuda")
        P = lambda t: t.data_ptr()
        # heads x n/64 x d x 6 bytes of split representatives: 700 x 2048 x 128 x 6 > 64 MiB
        # (only argument checks and the workspace plan run: nothing is launched)
        assert L.bsa_forward_noalloc(lib.handle, P(q), P(q), P(q), P(out), P(idx), 1, 700, 131072, 128, 1, 64,
                                     4, ctypes.c_float(0.1), 0, None) == m.BSA_ERR_UNSUPPORTED
        assert "fixed workspace" in m.bsa_last_error(lib.handle)
        assert L.bsa_forward_noalloc(lib.handle, P(q), P(q), P(q), P(out), P(idx), 1, 1, 100, 64, 1, 64,
                                     4, ctypes.c_float(0.1), 0, None) == m.BSA_ERR_UNSUPPORTED
        assert L.bsa_forward_noalloc(lib.handle, P(q), P(q), P(q), P(out), None, 1, 1, 128, 64, 1, 64,
                                     4, ctypes.c_float(0.1), 0, None) == m.BSA_ERR_INVALID_ARG
        torch.cuda.synchronize()
