"""GPU parity of variable-length batches (bsa_forward_varlen,
bsa_backward_varlen) against the fp64 oracle, through the C ABI.  Marked gpu.

Every sequence of a batch is its own attention problem, so the oracle runs on
each sequence alone ([1, heads, len, d] slices of the batch) and the GPU's rows
of that sequence must pass the same acceptance as bsa_forward's: indices
(numbered from the sequence's first block) bit-exact outside the tie band and
a valid top-k inside it, outputs within 1e-2 (bf16) / 1e-4 (fp32) of the
oracle's attention over the GPU's selection; gradients as in the backward
tests.  The lengths mix partial last blocks, whole blocks, a single row and an
empty sequence.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from test_gpu_parity import TOL, check_selection, say, use_strategy
from test_gpu_backward import TOLG, TOLL, close, single_key_rows

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

RAGGED = [1000, 64, 3000, 1, 0, 128, 4100, 257]
WHOLE = [1024, 64, 2048, 512, 192]


@pytest.fixture(scope="module")
def bsa():
    import content_dependent_block_amd as m
    lib = m.BlockSparseAttention(0)
    yield m, lib
    lib.close()


@pytest.fixture(autouse=True)
def _defaults(bsa):
    yield
    m, lib = bsa
    use_strategy(m, lib, "block_gather", "fused")


def strategy(m, lib, select, fine):
    use_strategy(m, lib, fine, select)


def dev_qkv(inp, dtype):
    """[1, h, total, d] host arrays -> [h, total, d] device tensors."""
    if dtype == "bf16":
        conv = lambda bits: torch.from_numpy(bits[0].view(np.int16)).view(torch.bfloat16).cuda()
        return conv(inp.q_bits), conv(inp.k_bits), conv(inp.v_bits)
    return tuple(torch.from_numpy(np.ascontiguousarray(x[0])).cuda() for x in (inp.q, inp.k, inp.v))


def seq_slice(x, cu, i):
    return np.ascontiguousarray(x[:, :, cu[i]:cu[i + 1]])


def forward_varlen(m, lib, w, inp, cu, topk, causal, head_topk=None):
    q, k, v = dev_qkv(inp, w.dtype)
    h, total, d = q.shape
    out = torch.empty((h, total, d), dtype=torch.float32, device="cuda")
    idx = torch.empty((h, total, topk), dtype=torch.int32, device="cuda")
    lse = torch.empty((h, total), dtype=torch.float32, device="cuda")
    m.bsa_forward_varlen(lib.handle, q, k, v, out, cu, idx, lse, topk=topk, head_topk=head_topk,
                         scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    return (q, k, v), out, idx, lse


def check_sequences(w, inp, cu, out, idx, topk, causal, head_topk=None):
    """Each sequence's rows against the oracle on that sequence alone."""
    out = out.cpu().numpy()
    idx = idx.cpu().numpy()
    h = inp.q.shape[1]
    worst = 0.0
    for i in range(cu.size - 1):
        n = int(cu[i + 1] - cu[i])
        if n == 0:
            continue
        q, k, v = (seq_slice(x, cu, i) for x in (inp.q, inp.k, inp.v))
        rows = np.arange(h * n, dtype=np.int64)
        s = oracle.scores(q, oracle.pool(k, w.block), w.block)
        gidx = idx[:, cu[i]:cu[i + 1]].reshape(h * n, topk)
        for hh in range(h):
            kh = topk if head_topk is None else int(head_topk[hh])
            sel = rows // n == hh
            oidx, kth, nxt = oracle.topk(s[sel], n, w.block, kh, causal, rows[sel])
            assert (gidx[sel, kh:] == -1).all()
            check_selection(gidx[sel, :kh], oidx, kth, nxt, s[sel], rows[sel], n, w.block, causal)
        ref = oracle.attend(q, k, v, gidx, w.block, causal, w.scale)
        err = float(np.abs(out[:, cu[i]:cu[i + 1]].reshape(h * n, -1) - ref).max())
        worst = max(worst, err)
        assert err <= TOL[w.dtype], f"sequence {i} (n = {n}): max|err| {err}"
    return worst


PATHS = [("fused", "block_gather"), ("panel", "block_gather"), ("fused", "query_tile"), ("fused", "query_tile16"),
         ("fused", "per_query")]


@pytest.mark.parametrize("select,fine", PATHS)
@pytest.mark.parametrize("name,causal,lengths", [
    ("dyn_bf16_n4k", False, RAGGED), ("dyn_bf16_n4k", True, RAGGED),
    ("tiny_fp32_n1k", False, RAGGED), ("tiny_fp32_n1k", True, WHOLE),
    ("dyn_bf16_n4k", True, WHOLE)])
def test_forward_varlen(bsa, select, fine, name, causal, lengths):
    m, lib = bsa
    strategy(m, lib, select, fine)
    w = W.WORKLOADS[name]
    inp, cu = W.generate_varlen(w, lengths, heads=2)
    say(f"[gpu] bsa_forward_varlen {name} causal={causal} {select}/{fine} lengths={lengths}")
    _, out, idx, _ = forward_varlen(m, lib, w, inp, cu, w.topk, causal)
    err = check_sequences(w, inp, cu, out, idx, w.topk, causal)
    say(f"    {cu.size - 1} sequences, max|err| = {err:.3g}")


@pytest.mark.parametrize("causal", [False, True])
def test_forward_varlen_d128_and_budgets(bsa, causal):
    """d = 128 rows, and per-head budgets: each head's rows keep their own k."""
    m, lib = bsa
    w = W.Workload("varlen_bf16_d128", 1, 3, 0, 128, "bf16", seed=11, topk=24, key_offsets=True)
    inp, cu = W.generate_varlen(w, [700, 2048, 65, 1500], heads=3)
    head_topk = [24, 3, 11]
    say(f"[gpu] bsa_forward_varlen d=128 causal={causal} budgets={head_topk}")
    _, out, idx, _ = forward_varlen(m, lib, w, inp, cu, 24, causal, head_topk=head_topk)
    check_sequences(w, inp, cu, out, idx, 24, causal, head_topk=head_topk)


@pytest.mark.parametrize("n", [4096, 1000])
def test_single_sequence_matches_bsa_forward(bsa, n):
    """One sequence: the same bits as bsa_forward on a [1, heads, n, d] batch."""
    m, lib = bsa
    w = W.WORKLOADS["dyn_bf16_n4k"]
    inp, cu = W.generate_varlen(w, [n], heads=4)
    say(f"[gpu] single-sequence varlen vs bsa_forward n={n}")
    (q, k, v), out, idx, lse = forward_varlen(m, lib, w, inp, cu, w.topk, True)
    out2 = torch.empty((1,) + tuple(out.shape), dtype=torch.float32, device="cuda")
    idx2 = torch.empty((1,) + tuple(idx.shape), dtype=torch.int32, device="cuda")
    lse2 = torch.empty((1,) + tuple(lse.shape), dtype=torch.float32, device="cuda")
    m.bsa_forward_train(lib.handle, q[None], k[None], v[None], out2, idx2, lse2, topk=w.topk,
                        scale=w.scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(idx2[0], idx)
    assert torch.equal(out2[0], out)
    assert torch.equal(lse2[0], lse)


@pytest.mark.parametrize("name,causal,lengths", [("dyn_bf16_n4k", True, RAGGED),
                                                 ("tiny_fp32_n1k", False, RAGGED),
                                                 ("dyn_bf16_n4k", False, WHOLE)])
def test_backward_varlen(bsa, name, causal, lengths):
    """Gradients of every sequence against the oracle's on that sequence, with
    the GPU forward's selection held fixed."""
    m, lib = bsa
    w = W.WORKLOADS[name]
    inp, cu = W.generate_varlen(w, lengths, heads=2)
    say(f"[gpu] bsa_backward_varlen {name} causal={causal} lengths={lengths}")
    qkv, out, idx, lse = forward_varlen(m, lib, w, inp, cu, w.topk, causal)
    h, total, d = out.shape
    dout = W.grad_output((h, total, d), w.seed)
    dq = torch.empty((h, total, d), dtype=torch.float32, device="cuda")
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    m.bsa_backward_varlen(lib.handle, *qkv, out, torch.from_numpy(dout).cuda(), idx, lse, dq, dk, dv, cu,
                          scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    gq, gk, gv = (x.cpu().numpy() for x in (dq, dk, dv))
    gidx = idx.cpu().numpy()
    glse = lse.cpu().numpy()
    for i in range(cu.size - 1):
        n = int(cu[i + 1] - cu[i])
        if n == 0:
            continue
        q, k, v = (seq_slice(x, cu, i) for x in (inp.q, inp.k, inp.v))
        sidx = gidx[:, cu[i]:cu[i + 1]].reshape(h * n, -1)
        sd = np.ascontiguousarray(dout[None, :, cu[i]:cu[i + 1]])
        rq, rl, rk, rv = oracle.attend_backward(q, k, v, sd, sidx, w.block, causal, w.scale)
        nb = -(-n // w.block)
        rk = rk.reshape(h, nb * w.block, d)[:, :n].reshape(h * n, d)
        rv = rv.reshape(h, nb * w.block, d)[:, :n].reshape(h * n, d)
        lerr = float(np.abs(glse[:, cu[i]:cu[i + 1]].reshape(-1) - rl).max())
        assert lerr <= TOLL[w.dtype], f"sequence {i}: lse max|err| {lerr}"
        one_row, one_key = single_key_rows(sidx, n, w.block, causal)
        floor = float(np.abs(rv).max())
        say(f"  sequence {i} (n = {n})")
        sl = slice(cu[i], cu[i + 1])
        close("dq", gq[:, sl].reshape(h * n, d), rq, TOLG[w.dtype], floor, one_row)
        close("dk", gk[:, sl].reshape(h * n, d), rk, TOLG[w.dtype], floor,
              one_key.reshape(h, nb * w.block)[:, :n].reshape(-1))
        close("dv", gv[:, sl].reshape(h * n, d), rv, TOLG[w.dtype])


def test_varlen_validation(bsa):
    """Malformed offsets and oversized batches are refused before any launch."""
    m, lib = bsa
    w = W.WORKLOADS["tiny_fp32_n1k"]
    inp, cu = W.generate_varlen(w, [100, 200], heads=1)
    q, k, v = dev_qkv(inp, w.dtype)
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    P = lambda t: None if t is None else t.data_ptr()

    def call(cu_arr, nseq, heads=1, d=64, topk=4):
        arr = None if cu_arr is None else np.ascontiguousarray(np.asarray(cu_arr, dtype=np.int32))
        ptr = None if arr is None else arr.ctypes.data
        return m._binding._lib.bsa_forward_varlen(lib.handle, P(q), P(k), P(v), P(out), None, None, ptr, nseq,
                                                   heads, d, m.BSA_FP32, 64, None, topk, w.scale, 0, None)

    assert call(cu, 2) == m.BSA_OK
    torch.cuda.synchronize()
    assert call(None, 2) == m.BSA_ERR_INVALID_ARG
    assert call([1, 100, 300], 2) == m.BSA_ERR_INVALID_ARG      # does not start at 0
    assert call([0, 200, 100], 2) == m.BSA_ERR_INVALID_ARG      # decreasing
    assert call([0, 0, 0], 2) == m.BSA_ERR_INVALID_ARG          # no rows
    assert call(cu, 0) == m.BSA_ERR_INVALID_ARG
    assert call(cu, 2, d=96) == m.BSA_ERR_UNSUPPORTED
    assert call(cu, 2, topk=0) == m.BSA_ERR_INVALID_ARG
    # 2049 blocks of whole-block sequences: refused before touching q
    assert call([0] + [64 * (i + 1) for i in range(2049)], 2049) == m.BSA_ERR_UNSUPPORTED
