"""GPU parity of the backward (bsa_forward_train + bsa_backward) against the
fp64 oracle (oracle.attend_backward), through the C ABI.  Marked gpu.

Acceptance (derived in the design notes from the arithmetic):
  * lse within 4e-3 absolute (bf16: the forward sums bf16-rounded weights,
    relative error <= 2^-9 of the sum) / 1e-5 (fp32);
  * dq, dk, dv: max |gpu - oracle| <= tol * max |oracle| per tensor, with tol
    1e-2 for bf16 inputs (P, dS and dout enter the MFMAs rounded to bf16) and
    1e-4 for fp32 inputs.  One exception: a query row that sees exactly one
    key has softmax weight 1, so its dq (and that key's share of dk) is 0 in
    exact arithmetic and the GPU leaves rounding residue of the size of the
    gradient's building blocks; for those rows of dq, and for the keys such a
    row sees in dk, the bound is tol * max(max |oracle|, max |dv|).
The isolated tests feed the backward the oracle's own selection, output and
lse; the end-to-end tests run the GPU forward and check its selection as the
forward tests do before comparing gradients on that selection.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOLG = {"bf16": 1e-2, "fp32": 1e-4}
TOLL = {"bf16": 4e-3, "fp32": 1e-5}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


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
    m.bsa_set_option(lib.handle, m.BSA_OPT_FINE_STRATEGY, m.BSA_FINE_BLOCK_GATHER)
    m.bsa_set_option(lib.handle, m.BSA_OPT_SELECT_STRATEGY, m.BSA_SELECT_FUSED)
    m.bsa_set_option(lib.handle, m.BSA_OPT_FINE_CHUNK_BYTES, 1 << 30)


def to_dev(inp, dtype):
    if dtype == "bf16":
        conv = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
        return conv(inp.q_bits), conv(inp.k_bits), conv(inp.v_bits)
    return (torch.from_numpy(inp.q).cuda(), torch.from_numpy(inp.k).cuda(),
            torch.from_numpy(inp.v).cuda())


def close(name, g, ref, tol, floor=0.0, floor_rows=None):
    """max|g - ref| <= tol * max|ref| on every row; rows flagged in
    floor_rows (a row that sees a single key, or a key seen by such a row)
    may instead reach tol * max(max|ref|, floor): their exact value cancels
    to 0 and the GPU leaves rounding residue of the building blocks' size."""
    g = np.asarray(g).reshape(ref.shape[0], -1)
    ref = np.asarray(ref).reshape(ref.shape[0], -1)
    row_err = np.abs(g - ref).max(axis=1) if ref.size else np.zeros(0)
    top = float(np.abs(ref).max()) if ref.size else 0.0
    flagged = np.zeros(ref.shape[0], dtype=bool) if floor_rows is None else np.asarray(floor_rows, bool)
    plain = float(row_err[~flagged].max()) if (~flagged).any() else 0.0
    cancel = float(row_err[flagged].max()) if flagged.any() else 0.0
    say(f"    {name}: max|err| = {plain:.3g} (rows with one visible key: {cancel:.3g}, "
        f"{int(flagged.sum())} of them), max|ref| = {top:.3g}, ratio {plain / max(top, 1e-30):.3g}")
    assert plain <= tol * top, f"{name}: {plain} > {tol} * {top}"
    assert cancel <= tol * max(top, floor), f"{name} (one-key rows): {cancel} > {tol} * max({top}, {floor})"


def single_key_rows(idx, n, block, causal):
    """For every query row of idx ([bh*n, topk], -1 padded): does it see
    exactly one key?  Also the padded-key mask [bh, nb*block] of the keys such
    rows see (the first key of their only block with a visible key)."""
    idx = np.asarray(idx).reshape(-1, idx.shape[-1]).astype(np.int64)
    rows = np.arange(idx.shape[0])
    i = rows % n
    qb = i // block
    nb = -(-n // block)
    valid = (idx >= 0) & (idx < nb)
    beta = np.where(valid, idx, 0)
    per = np.minimum(block, n - beta * block)          # keys of the block (a ragged last block has fewer)
    if causal:
        per = np.where(beta == qb[:, None], np.minimum(per, i[:, None] % block + 1), per)
        per = np.where(beta > qb[:, None], 0, per)
    per = np.where(valid, per, 0)
    one = per.sum(axis=1) == 1
    keys = np.zeros((idx.shape[0] // n, nb * block), dtype=bool)
    r1 = np.nonzero(one)[0]
    if r1.size:
        b1 = beta[r1, np.argmax(per[r1] > 0, axis=1)]
        keys[r1 // n, b1 * block] = True
    return one, keys


def gpu_backward(m, lib, qkv, out, dout, idx, lse, scale, causal):
    q = qkv[0]
    dq = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    m.bsa_backward(lib.handle, *qkv, out, dout, idx, lse, dq, dk, dv, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()


def oracle_selection(inp, w, topk, causal, head_topk=None):
    b, h, n, d = inp.q.shape
    r = oracle.pool(inp.k, w.block)
    s = oracle.scores(inp.q, r, w.block)
    if head_topk is None:
        idx, kth, nxt = oracle.topk(s, n, w.block, topk, causal)
        return idx, kth, nxt, s
    idx = np.full((b * h * n, topk), -1, np.int32)
    kth = np.empty(b * h * n)
    nxt = np.empty(b * h * n)
    rows = np.arange(b * h * n)
    for hh in range(h):
        sel = (rows // n) % h == hh
        i, a, c = oracle.topk(s[sel], n, w.block, head_topk[hh], causal, rows[sel])
        idx[sel, :head_topk[hh]] = i
        kth[sel], nxt[sel] = a, c
    return idx, kth, nxt, s


def compare_grads(w, inp, dout, idx, g, causal, scale, rows=None, blocks=None):
    b, h, n, d = inp.q.shape
    dq, lse, dk, dv = oracle.attend_backward(inp.q, inp.k, inp.v, dout, idx, w.block, causal, scale,
                                             rows=rows, key_blocks=blocks)
    gq, gk, gv = (x.reshape(-1, d) for x in g)
    if rows is not None:
        gq = gq[rows]
    nb = n // w.block
    if blocks is None:
        blocks = np.arange(b * h * nb)
    keys = (blocks[:, None] * w.block + np.arange(w.block)[None, :]).reshape(-1)
    floor = float(np.abs(dv).max())
    one_row, one_key = single_key_rows(idx, n, w.block, causal)
    rsel = np.arange(b * h * n) if rows is None else rows
    close("dq", gq, dq, TOLG[w.dtype], floor, one_row[rsel])
    close("dk", gk[keys], dk.reshape(-1, d), TOLG[w.dtype], floor, one_key.reshape(-1)[keys])
    close("dv", gv[keys], dv.reshape(-1, d), TOLG[w.dtype])
    return lse


# ------------------------------------------------ backward in isolation --
@pytest.mark.parametrize("name,causal,topk", [("tiny_fp32_n1k", False, 4), ("tiny_fp32_n1k", True, 4),
                                              ("dyn_bf16_n4k", False, 16), ("dyn_bf16_n4k", True, 16),
                                              ("dyn_bf16_n4k", False, 1), ("tiny_fp32_n1k", False, 16)])
def test_backward_on_oracle_inputs(bsa, name, causal, topk):
    """bsa_backward on the oracle's selection, output and lse: the gradients
    match the oracle's over all rows and all key blocks."""
    m, lib = bsa
    w = W.WORKLOADS[name]
    inp = W.generate(w)
    b, h, n, d = inp.q.shape
    say(f"[gpu] bsa_backward on oracle inputs {name} causal={causal} k={topk}")
    idx, _, _, _ = oracle_selection(inp, w, topk, causal)
    out = oracle.attend(inp.q, inp.k, inp.v, idx, w.block, causal, w.scale)
    dout = W.grad_output(inp.q.shape, w.seed)
    _, lse, _, _ = oracle.attend_backward(inp.q, inp.k, inp.v, dout, idx, w.block, causal, w.scale,
                                          key_blocks=np.zeros(0, np.int64))
    dev = lambda x, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(x)).to(dt).cuda()
    g = gpu_backward(m, lib, to_dev(inp, w.dtype), dev(out.reshape(inp.q.shape)), dev(dout),
                     dev(idx.reshape(b, h, n, topk), torch.int32), dev(lse.reshape(b, h, n)),
                     w.scale, causal)
    compare_grads(w, inp, dout, idx, g, causal, w.scale)


# ---------------------------------------------------------- end to end --
def forward_train(m, lib, w, inp, topk, causal, head_topk=None):
    b, h, n, d = inp.q.shape
    qkv = to_dev(inp, w.dtype)
    out = torch.empty((b, h, n, d), dtype=torch.float32, device="cuda")
    idx = torch.empty((b, h, n, topk), dtype=torch.int32, device="cuda")
    lse = torch.empty((b, h, n), dtype=torch.float32, device="cuda")
    m.bsa_forward_train(lib.handle, *qkv, out, idx, lse, topk=topk, head_topk=head_topk,
                        scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    return qkv, out, idx, lse


def check_selection(gidx, oidx, kth, nxt):
    fin = np.isfinite(kth) & np.isfinite(nxt)
    band = np.zeros(kth.size, bool)
    band[fin] = np.abs(kth[fin] - nxt[fin]) <= 1e-4 * np.maximum(np.abs(kth[fin]), np.abs(nxt[fin]))
    bad = ~(gidx == oidx).all(axis=1) & ~band
    assert not bad.any(), f"{bad.sum()} rows select other blocks outside the tie band"


@pytest.mark.parametrize("fine", ["block_gather", "query_tile", "per_query"])
@pytest.mark.parametrize("name,causal,topk,head_topk", [
    ("tiny_fp32_n1k", False, 4, None), ("tiny_fp32_n1k", True, 4, None),
    ("dyn_bf16_n4k", False, 16, None), ("dyn_bf16_n4k", True, 16, None),
    ("dyn_bf16_n4k", True, 32, [1, 3, 16, 7, 32, 2, 9, 16]),
])
def test_forward_train_and_backward(bsa, fine, name, causal, topk, head_topk):
    """bsa_forward_train's selection (as in the forward tests), output and
    lse against the oracle, then bsa_backward's gradients on that selection."""
    m, lib = bsa
    m.bsa_set_option(lib.handle, m.BSA_OPT_FINE_STRATEGY,
                     {"block_gather": m.BSA_FINE_BLOCK_GATHER, "query_tile": m.BSA_FINE_QUERY_TILE,
                      "per_query": m.BSA_FINE_PER_QUERY}[fine])
    w = W.WORKLOADS[name]
    inp = W.generate(w)
    b, h, n, d = inp.q.shape
    say(f"[gpu] forward_train + backward {name} causal={causal} k={topk} budgets={head_topk} fine={fine}")
    qkv, out, idx, lse = forward_train(m, lib, w, inp, topk, causal, head_topk)
    gidx = idx.cpu().numpy().reshape(-1, topk)
    oidx, kth, nxt, _ = oracle_selection(inp, w, topk, causal, head_topk)
    check_selection(gidx, oidx, kth, nxt)
    ref_out = oracle.attend(inp.q, inp.k, inp.v, gidx, w.block, causal, w.scale)
    err = np.abs(out.cpu().numpy().reshape(-1, d) - ref_out).max()
    assert err <= {"bf16": 1e-2, "fp32": 1e-4}[w.dtype], err
    dout = W.grad_output(inp.q.shape, w.seed)
    g = gpu_backward(m, lib, qkv, out, torch.from_numpy(dout).cuda(), idx, lse, w.scale, causal)
    ref_lse = compare_grads(w, inp, dout, gidx, g, causal, w.scale)
    lerr = np.abs(lse.cpu().numpy().reshape(-1) - ref_lse).max()
    say(f"    lse: max|err| = {lerr:.3g}")
    assert lerr <= TOLL[w.dtype]


@pytest.mark.parametrize("name,n,topk,causal", [("tiny_fp32_n1k", 1000, 4, False),
                                                 ("tiny_fp32_n1k", 1000, 4, True),
                                                 ("dyn_bf16_n4k", 4100, 16, True),
                                                 ("dyn_bf16_n4k", 65, 16, False),
                                                 ("tiny_fp32_n1k", 1, 4, True)])
def test_backward_ragged_n(bsa, name, n, topk, causal):
    """n not a multiple of 64: gradients of the padded keys never reach the
    caller and the last block's valid keys get theirs; all rows, all keys."""
    m, lib = bsa
    w = W.WORKLOADS[name]
    inp = W.generate(w, n=n)
    say(f"[gpu] forward_train + backward ragged {name} n={n} k={topk} causal={causal}")
    qkv, out, idx, lse = forward_train(m, lib, w, inp, topk, causal)
    gidx = idx.cpu().numpy().reshape(-1, topk)
    oidx, kth, nxt, _ = oracle_selection(inp, w, topk, causal)
    check_selection(gidx, oidx, kth, nxt)
    dout = W.grad_output(inp.q.shape, w.seed)
    g = gpu_backward(m, lib, qkv, out, torch.from_numpy(dout).cuda(), idx, lse, w.scale, causal)
    dq, ref_lse, dk, dv = oracle.attend_backward(inp.q, inp.k, inp.v, dout, gidx, w.block, causal, w.scale)
    d = w.d
    floor = float(np.abs(dv).max())
    one_row, one_key = single_key_rows(gidx, n, w.block, causal)
    close("dq", g[0].reshape(-1, d), dq, TOLG[w.dtype], floor, one_row)
    b, h = inp.q.shape[:2]
    nb = -(-n // w.block)
    # oracle dk/dv are per block of 64 rows (rows past n are zero): keep the valid ones
    keep = (np.arange(nb * w.block) < n)
    close("dk", g[1].reshape(-1, d), dk.reshape(b * h, nb * w.block, d)[:, keep].reshape(-1, d), TOLG[w.dtype],
          floor, one_key[:, keep].reshape(-1))
    close("dv", g[2].reshape(-1, d), dv.reshape(b * h, nb * w.block, d)[:, keep].reshape(-1, d), TOLG[w.dtype])
    assert np.abs(lse.cpu().numpy().reshape(-1) - ref_lse).max() <= TOLL[w.dtype]


def test_backward_d128_causal(bsa):
    """d = 128 (the long causal workload's head size) at n = 4096, 2 heads, k = 32."""
    m, lib = bsa
    w = W.WORKLOADS["causal_bf16_n128k"]
    inp = W.generate(w, n=4096, heads=2)
    b, h, n, d = inp.q.shape
    say(f"[gpu] backward d=128 causal n={n} heads={h} k={w.topk}")
    qkv, out, idx, lse = forward_train(m, lib, w, inp, w.topk, True)
    dout = W.grad_output(inp.q.shape, w.seed)
    g = gpu_backward(m, lib, qkv, out, torch.from_numpy(dout).cuda(), idx, lse, w.scale, True)
    compare_grads(w, inp, dout, idx.cpu().numpy().reshape(-1, w.topk), g, True, w.scale)


def test_backward_fp32_d128(bsa):
    m, lib = bsa
    w = W.WORKLOADS["tiny_fp32_n1k"]
    rng = np.random.default_rng(77)
    q, k, v = (rng.standard_normal((1, 2, 1024, 128), dtype=np.float32) for _ in range(3))
    inp = W.Inputs(q, k, v)
    say("[gpu] backward fp32 d=128 n=1024 heads=2 k=5")
    qkv, out, idx, lse = forward_train(m, lib, w, inp, 5, False)
    dout = W.grad_output(q.shape, 77)
    g = gpu_backward(m, lib, qkv, out, torch.from_numpy(dout).cuda(), idx, lse, w.scale, False)
    compare_grads(w, inp, dout, idx.cpu().numpy().reshape(-1, 5), g, False, w.scale)


def test_backward_headline_sampled(bsa):
    """The 32k workload: dq on sampled rows and dk, dv on sampled key blocks
    against the oracle, plus the identity sum_j dv_j = sum_i dout_i per head
    over the full output."""
    m, lib = bsa
    w = W.WORKLOADS["dyn_bf16_n32k"]
    inp = W.generate(w)
    b, h, n, d = inp.q.shape
    say(f"[gpu] backward headline n={n} heads={h} k={w.topk}")
    qkv, out, idx, lse = forward_train(m, lib, w, inp, w.topk, w.causal)
    dout = W.grad_output(inp.q.shape, w.seed)
    g = gpu_backward(m, lib, qkv, out, torch.from_numpy(dout).cuda(), idx, lse, w.scale, w.causal)
    rng = np.random.default_rng(9)
    rows = np.sort(rng.choice(b * h * n, 1500, replace=False))
    blocks = np.sort(rng.choice(b * h * (n // 64), 12, replace=False))
    compare_grads(w, inp, dout, idx.cpu().numpy().reshape(-1, w.topk), g, w.causal, w.scale,
                  rows=rows, blocks=blocks)
    dv_sum = g[2].reshape(b * h, n, d).astype(np.float64).sum(axis=1)
    do_sum = dout.reshape(b * h, n, d).astype(np.float64).sum(axis=1)
    err = np.abs(dv_sum - do_sum).max()
    say(f"    sum dv vs sum dout: max|err| = {err:.3g} (max {np.abs(do_sum).max():.3g})")
    assert err <= 1e-2 * np.abs(do_sum).max()


def test_backward_causal_long_sampled(bsa):
    """The long causal workload at full size (8 x 131072 x 128, k = 32): the
    dq rows span eight row chunks, so dk and dv are summed across chunks.
    dq on sampled rows, dk and dv on sampled key blocks of the later half of
    the sequence (fewer rows select them, which keeps the oracle short)."""
    m, lib = bsa
    w = W.WORKLOADS["causal_bf16_n128k"]
    inp = W.generate(w)
    b, h, n, d = inp.q.shape
    say(f"[gpu] backward causal long n={n} heads={h} d={d} k={w.topk}")
    qkv, out, idx, lse = forward_train(m, lib, w, inp, w.topk, True)
    dout = W.grad_output(inp.q.shape, w.seed)
    g = gpu_backward(m, lib, qkv, out, torch.from_numpy(dout).cuda(), idx, lse, w.scale, True)
    del qkv, out, lse
    rng = np.random.default_rng(13)
    rows = np.sort(rng.choice(b * h * n, 400, replace=False))
    nb = n // w.block
    heads = rng.integers(0, b * h, size=3)
    blocks = np.sort(heads * nb + rng.integers(nb // 2, nb, size=3))
    compare_grads(w, inp, dout, idx.cpu().numpy().reshape(-1, w.topk), g, True, w.scale,
                  rows=rows, blocks=blocks)


def test_backward_deterministic_and_chunked(bsa):
    """Two calls give identical dq bits and dk, dv equal within rounding (the
    order of a block's pairs comes from the bucketing's atomics); a small row
    chunk (several chunks per head) gives identical dq and dk, dv within
    rounding."""
    m, lib = bsa
    w = W.WORKLOADS["dyn_bf16_n4k"]
    inp = W.generate(w)
    say("[gpu] backward determinism and chunking")
    qkv, out, idx, lse = forward_train(m, lib, w, inp, 16, True)
    dout = torch.from_numpy(W.grad_output(inp.q.shape, w.seed)).cuda()
    a = gpu_backward(m, lib, qkv, out, dout, idx, lse, w.scale, True)
    b = gpu_backward(m, lib, qkv, out, dout, idx, lse, w.scale, True)
    assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32))
    for x, y in zip(a[1:], b[1:]):
        assert np.abs(x - y).max() <= 1e-5 * np.abs(x).max()
    m.bsa_set_option(lib.handle, m.BSA_OPT_FINE_CHUNK_BYTES, 3000 * 16 * (64 * 4 + 8))
    c = gpu_backward(m, lib, qkv, out, dout, idx, lse, w.scale, True)
    assert np.array_equal(a[0], c[0])
    for x, y in zip(a[1:], c[1:]):
        assert np.abs(x - y).max() <= 1e-5 * np.abs(x).max()


def test_autograd_function(bsa):
    """block_sparse_attention under torch autograd returns the same gradients
    as the C ABI calls."""
    m, lib = bsa
    w = W.WORKLOADS["dyn_bf16_n4k"]
    inp = W.generate(w)
    say("[gpu] autograd function")
    qkv = [t.clone().requires_grad_(True) for t in to_dev(inp, w.dtype)]
    out = m.block_sparse_attention(*qkv, 16, lib=lib, causal=True)
    dout = torch.from_numpy(W.grad_output(inp.q.shape, w.seed)).cuda()
    (out * dout).sum().backward()
    qkv2, out2, idx, lse = forward_train(m, lib, w, inp, 16, True)
    ref = gpu_backward(m, lib, qkv2, out2, dout, idx, lse, w.scale, True)
    for i, (t, r) in enumerate(zip(qkv, ref)):
        assert t.grad.dtype == torch.bfloat16
        got = t.grad.float().cpu().numpy()
        want = torch.from_numpy(r).to(torch.bfloat16).float().numpy()
        if i == 0:   # dq: the same bits on every call
            np.testing.assert_array_equal(got, want)
        else:        # dk, dv: equal within rounding, so within one bf16 step
            assert (np.abs(got - want) <= 2.0 ** -7 * np.abs(want) + 1e-6).all()


def test_backward_validation(bsa):
    m, lib = bsa
    L = m._binding._lib
    h = lib.handle
    say("[gpu] backward validation statuses")
    q = torch.zeros((1, 1, 128, 64), dtype=torch.bfloat16, device="cuda")
    f = torch.zeros((1, 1, 128, 64), dtype=torch.float32, device="cuda")
    idx = torch.zeros((1, 1, 128, 2), dtype=torch.int32, device="cuda")
    lse = torch.zeros((1, 1, 128), dtype=torch.float32, device="cuda")
    P = lambda t: None if t is None else t.data_ptr()

    def bwd(**kw):
        a = dict(q=P(q), out=P(f), dout=P(f), idx=P(idx), lse=P(lse), dq=P(f), n=128, topk=2, scale=0.125)
        a.update(kw)
        return L.bsa_backward(h, a["q"], a["q"], a["q"], a["out"], a["dout"], a["idx"], a["lse"], a["dq"],
                              a["dq"], a["dq"], 1, 1, a["n"], 64, 1, 64, a["topk"], a["scale"], 0, None)
    assert bwd() == m.BSA_OK
    for key in ("q", "out", "dout", "idx", "lse", "dq"):
        assert bwd(**{key: None}) == m.BSA_ERR_INVALID_ARG, key
    assert bwd(dq=P(f) + 4) == m.BSA_ERR_INVALID_ARG
    assert bwd(topk=0) == m.BSA_ERR_INVALID_ARG
    assert bwd(scale=0.0) == m.BSA_ERR_INVALID_ARG
    assert bwd(n=100) == m.BSA_OK                  # ragged n: padded internally
    assert bwd(n=64 * 2049) == m.BSA_ERR_UNSUPPORTED

    def fwd(**kw):
        a = dict(idx=P(idx), lse=P(lse), ks=None, topk=2)
        a.update(kw)
        return L.bsa_forward_train(h, P(q), P(q), P(q), P(f), a["idx"], a["lse"], 1, 1, 128, 64, 1, 64,
                                   a["ks"], a["topk"], 0.125, 0, None)
    assert fwd() == m.BSA_OK
    assert fwd(idx=None) == m.BSA_ERR_INVALID_ARG
    assert fwd(lse=None) == m.BSA_ERR_INVALID_ARG
    bad = np.array([3], np.int32)
    assert fwd(ks=bad.ctypes.data) == m.BSA_ERR_INVALID_ARG
    good = np.array([1], np.int32)
    assert fwd(ks=good.ctypes.data) == m.BSA_OK
    torch.cuda.synchronize()
