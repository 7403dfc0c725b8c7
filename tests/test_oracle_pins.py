"""Pins of the fp64 oracle to things other than itself: closed forms, textbook
routines (dense attention), brute force on tiny inputs, hand-worked examples
and the numbers the pages print.  Each test names the oracle function it pins
and the passage it follows.  CPU only."""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _dense_attention(q, k, v, scale, mask=None):
    """Textbook softmax attention (numpy, fp64) for one head [n, d]."""
    z = (q.astype(np.float64) @ k.astype(np.float64).T) * scale
    if mask is not None:
        z = np.where(mask, z, -np.inf)
    zmax = np.max(z, axis=1, keepdims=True)
    zmax = np.where(np.isfinite(zmax), zmax, 0.0)
    w = np.exp(z - zmax)
    den = w.sum(axis=1, keepdims=True)
    out = (w @ v.astype(np.float64))
    return np.where(den > 0, out / np.where(den > 0, den, 1.0), 0.0)


# ---------------------------------------------------------------- pooling --
def test_pool_column_sums():
    """oracle.pool: block means times block sizes add back to the key column
    sums (mean-pooling, 'Two-stage block indexer'); includes a partial block."""
    rng = np.random.default_rng(10)
    for n, B in [(256, 64), (200, 64), (7, 3)]:
        k = rng.standard_normal((3, n, 8)).astype(np.float32)
        r = oracle.pool(k, B)
        nb = -(-n // B)
        counts = np.array([min(B, n - b * B) for b in range(nb)], dtype=np.float64)
        lhs = (r * counts[None, :, None]).sum(axis=1)
        rhs = k.astype(np.float64).sum(axis=1)
        np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-12)


def test_pool_hand_example():
    """oracle.pool on a 4x2 example worked by hand: blocks {0,1} and {2,3}."""
    k = np.array([[[1, 2], [3, 4], [5, 6], [7, 8]]], dtype=np.float32)
    np.testing.assert_array_equal(oracle.pool(k, 2)[0], [[2, 3], [6, 7]])


# ----------------------------------------------------------------- scores --
def test_scores_are_a_matrix_product():
    """oracle.scores equals Q @ R^T computed by numpy's matmul (Stage 1 scores
    every query against every block representative)."""
    rng = np.random.default_rng(11)
    q = rng.standard_normal((2, 96, 16)).astype(np.float32)
    k = rng.standard_normal((2, 96, 16)).astype(np.float32)
    r = oracle.pool(k, 32)
    s = oracle.scores(q, r, 32)
    ref = np.concatenate([q[h].astype(np.float64) @ r[h].T for h in range(2)])
    np.testing.assert_allclose(s, ref, rtol=1e-13, atol=1e-13)


# -------------------------------------------------------------- selection --
def _rank_select(row, k, allowed, forced=None):
    """Brute-force selection by pairwise rank: block b is kept iff fewer than
    k allowed blocks beat it (higher score, or equal score and lower index);
    a forced block beats everything."""
    def beats(g, b):
        if forced is not None and g == forced:
            return b != forced
        if forced is not None and b == forced:
            return False
        return row[g] > row[b] or (row[g] == row[b] and g < b)
    keff = min(k, len(allowed))
    sel = sorted(b for b in allowed if sum(beats(g, b) for g in allowed if g != b) < keff)
    return sel + [-1] * (k - len(sel))


def test_topk_matches_pairwise_rank_with_ties():
    """oracle.topk against the rank definition, with many exact ties
    (scores rounded to one decimal); ties go to the lower index."""
    rng = np.random.default_rng(12)
    s = np.round(rng.standard_normal((300, 16)), 1)
    idx, _, _ = oracle.topk(s, n=16 * 64, block=64, k=4, causal=False)
    for r in range(s.shape[0]):
        assert list(idx[r]) == _rank_select(s[r], 4, list(range(16)))


def test_topk_is_the_max_sum_subset():
    """oracle.topk on the 16-block, k=4 shape: with distinct scores the kept
    set is the 4-subset of largest total score (enumerate all 1820)."""
    rng = np.random.default_rng(13)
    s = rng.standard_normal((40, 16))
    idx, kth, nxt = oracle.topk(s, n=1024, block=64, k=4, causal=False)
    subsets = np.array(list(itertools.combinations(range(16), 4)))
    for r in range(s.shape[0]):
        best = subsets[np.argmax(s[r][subsets].sum(axis=1))]
        assert list(idx[r]) == sorted(best.tolist())
        order = np.sort(s[r])[::-1]
        assert kth[r] == order[3] and nxt[r] == order[4]


def test_topk_signed_zero_and_exact_ties():
    """-0 and +0 tie, and the lower index wins (constructed row)."""
    s = np.array([[-0.0, 0.0, -1.0, 0.0, -0.0, -2.0]])
    idx, _, _ = oracle.topk(s, n=6 * 4, block=4, k=3, causal=False)
    assert list(idx[0]) == [0, 1, 3]


def test_topk_clamps_and_pads():
    """k larger than the number of blocks keeps every block, ascending, and
    pads with -1."""
    s = np.array([[3.0, 1.0, 2.0]])
    idx, kth, nxt = oracle.topk(s, n=12, block=4, k=5, causal=False)
    assert list(idx[0]) == [0, 1, 2, -1, -1]
    assert kth[0] == 1.0 and math.isnan(nxt[0])


def test_topk_causal_against_rank():
    """Causal variant: candidates are blocks <= the query's block and the own
    block is always kept (brute-force rank with a forced element)."""
    rng = np.random.default_rng(14)
    n, B, k = 16 * 8, 8, 3
    rows = np.arange(n, dtype=np.int64)
    s = np.round(rng.standard_normal((n, 16)), 1)
    idx, _, _ = oracle.topk(s, n=n, block=B, k=k, causal=True, rows=rows)
    for r in range(n):
        qb = r // B
        assert list(idx[r]) == _rank_select(s[r], k, list(range(qb + 1)), forced=qb)


# -------------------------------------------------------- fine attention --
def test_attend_equals_dense_when_every_block_is_kept():
    """k*B >= N keeps every block, so the fine stage is dense softmax
    attention (textbook, numpy)."""
    rng = np.random.default_rng(15)
    bh, n, d, B = 2, 256, 32, 64
    q, k, v = (rng.standard_normal((bh, n, d)).astype(np.float32) for _ in range(3))
    out, idx, _, _ = oracle.forward(q, k, v, block=B, topk_=4, causal=False, scale=0.3)
    assert (idx == np.arange(4)).all()
    ref = np.concatenate([_dense_attention(q[h], k[h], v[h], 0.3) for h in range(bh)])
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_attend_equals_dense_causal():
    """Causal with k >= number of blocks: dense causal attention."""
    rng = np.random.default_rng(16)
    n, d, B = 192, 16, 32
    q, k, v = (rng.standard_normal((1, n, d)).astype(np.float32) for _ in range(3))
    out, idx, _, _ = oracle.forward(q, k, v, block=B, topk_=8, causal=True, scale=0.25)
    for i in range(n):
        qb = i // B
        assert list(idx[i][: qb + 1]) == list(range(qb + 1))
        assert (idx[i][qb + 1:] == -1).all()
    ref = _dense_attention(q[0], k[0], v[0], 0.25, mask=np.tril(np.ones((n, n), bool)))
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_attend_single_block():
    """k = 1: attention within the one selected block (numpy on the slice)."""
    rng = np.random.default_rng(17)
    n, d, B = 256, 16, 64
    q, k, v = (rng.standard_normal((1, n, d)).astype(np.float32) for _ in range(3))
    idx = rng.integers(0, n // B, size=(n, 1)).astype(np.int32)
    out = oracle.attend(q, k, v, idx, block=B, causal=False, scale=0.5)
    for i in range(0, n, 7):
        b = idx[i, 0]
        sl = slice(b * B, b * B + B)
        ref = _dense_attention(q[0, i:i + 1], k[0, sl], v[0, sl], 0.5)
        np.testing.assert_allclose(out[i], ref[0], rtol=1e-12, atol=1e-12)


def test_attend_invariants():
    """V constant -> output constant; scale 0 -> plain mean of the visible
    values; block order in the index list does not matter."""
    rng = np.random.default_rng(18)
    n, d, B, k = 512, 8, 64, 3
    q, kk = (rng.standard_normal((1, n, d)).astype(np.float32) for _ in range(2))
    idx = np.stack([rng.choice(n // B, size=k, replace=False) for _ in range(n)]).astype(np.int32)
    vconst = np.full((1, n, d), 1.75, dtype=np.float32)
    out = oracle.attend(q, kk, vconst, idx, block=B, causal=False, scale=0.4)
    np.testing.assert_allclose(out, 1.75, rtol=1e-14)
    v = rng.standard_normal((1, n, d)).astype(np.float32)
    out0 = oracle.attend(q, kk, v, idx, block=B, causal=False, scale=0.0)
    for i in range(0, n, 13):
        keys = np.concatenate([np.arange(b * B, b * B + B) for b in idx[i]])
        np.testing.assert_allclose(out0[i], v[0, keys].astype(np.float64).mean(axis=0),
                                   rtol=1e-12, atol=1e-12)
    perm = idx[:, ::-1].copy()
    np.testing.assert_allclose(oracle.attend(q, kk, v, perm, block=B, causal=False, scale=0.4),
                               oracle.attend(q, kk, v, idx, block=B, causal=False, scale=0.4),
                               rtol=1e-12, atol=1e-12)


def test_forward_hand_worked_example():
    """Both stages on a 4-token example worked by hand (B=2, k=1, scale=1).
    K blocks {[2,0],[0,0]} and {[0,1],[0,3]} pool to [1,0] and [0,2]."""
    q = np.array([[[2, 1], [0, 3], [1, -1], [-1, 0]]], dtype=np.float32)
    k = np.array([[[2, 0], [0, 0], [0, 1], [0, 3]]], dtype=np.float32)
    v = np.array([[[1, 0], [0, 1], [2, 2], [4, 0]]], dtype=np.float32)
    out, idx, kth, nxt = oracle.forward(q, k, v, block=2, topk_=1, causal=False, scale=1.0)
    # scores: row0 [2,2] tie -> 0; row1 [0,6] -> 1; row2 [1,-2] -> 0; row3 [-1,0] -> 1
    assert idx[:, 0].tolist() == [0, 1, 0, 1]
    assert kth.tolist() == [2, 6, 1, 0] and nxt.tolist() == [2, 0, -2, -1]
    e = math.exp
    V = v[0].astype(np.float64)
    want = np.array([
        (e(4) * V[0] + V[1]) / (e(4) + 1),            # z = [4, 0]
        (e(3) * V[2] + e(9) * V[3]) / (e(3) + e(9)),  # z = [3, 9]
        (e(2) * V[0] + V[1]) / (e(2) + 1),            # z = [2, 0]
        (V[2] + V[3]) / 2,                            # z = [0, 0]
    ])
    np.testing.assert_allclose(out, want, rtol=1e-14)


def test_forward_hand_worked_causal():
    """Causal variant of the same example: own block forced, keys j <= i."""
    q = np.array([[[2, 1], [0, 3], [1, -1], [-1, 0]]], dtype=np.float32)
    k = np.array([[[2, 0], [0, 0], [0, 1], [0, 3]]], dtype=np.float32)
    v = np.array([[[1, 0], [0, 1], [2, 2], [4, 0]]], dtype=np.float32)
    out, idx, _, _ = oracle.forward(q, k, v, block=2, topk_=1, causal=True, scale=1.0)
    assert idx[:, 0].tolist() == [0, 0, 1, 1]
    e = math.exp
    V = v[0].astype(np.float64)
    want = np.array([
        V[0],                                         # only key 0 visible
        (V[0] + V[1]) / 2,                            # q1.k0 = q1.k1 = 0
        V[2],                                         # block 1, key 2 only
        (V[2] + V[3]) / 2,                            # q3.k2 = q3.k3 = 0
    ])
    np.testing.assert_allclose(out, want, rtol=1e-14)
    # and with k = 2 row 3 sees all four keys: z = [-2, 0, 0, 0]
    out2, idx2, _, _ = oracle.forward(q, k, v, block=2, topk_=2, causal=True, scale=1.0)
    assert idx2[3].tolist() == [0, 1]
    w = np.array([e(-2), 1, 1, 1])
    np.testing.assert_allclose(out2[3], (w[:, None] * V).sum(0) / w.sum(), rtol=1e-14)


# --------------------------------------------------------- static pattern --
def test_window_stride_mask_small_hand_case():
    """The [P2] pattern on n=8, w=1, s=4, compared with the mask written out
    by hand in the golden file."""
    g = _load("static_pattern_counts.json")["small_case"]
    m = oracle.window_stride_mask(g["n"], g["window"], g["stride"])
    want = np.array([[int(c) for c in row] for row in g["mask_rows"]], dtype=np.uint8)
    np.testing.assert_array_equal(m, want)


def test_window_stride_counts_closed_form():
    """Pairs and 64x64 tiles of the n=8192, w=32, s=512 pattern match the
    closed-form counts derived in the golden file."""
    g = _load("static_pattern_counts.json")
    m = oracle.window_stride_mask(g["n"], g["window"], g["stride"])
    assert int(m.sum(dtype=np.int64)) == g["active_pairs"]
    t = g["tile"]
    tiles = m.reshape(g["n"] // t, t, g["n"] // t, t).any(axis=(1, 3))
    assert int(tiles.sum()) == g["active_tiles"]


def test_attend_mask_equals_dense_masked():
    """oracle.attend_mask against textbook masked softmax attention (masked
    logits are -inf); an all-masked row gives zeros."""
    rng = np.random.default_rng(19)
    n, d = 96, 16
    q, k, v = (rng.standard_normal((2, n, d)).astype(np.float32) for _ in range(3))
    mask = rng.random((n, n)) < 0.2
    mask[5, :] = False
    out = oracle.attend_mask(q, k, v, mask.astype(np.uint8), 0.3)
    ref = np.concatenate([_dense_attention(q[h], k[h], v[h], 0.3, mask=mask) for h in range(2)])
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    assert (out[5] == 0).all() and (out[n + 5] == 0).all()


# ------------------------------------------------------------ FLOP counts --
def test_flop_counts_reproduce_the_page():
    """At N=32768, H=8, D=64, B=64, k=16 the page prints 87.2B sparse vs 2.24T
    dense FLOPs (3.9%) and 1024 attended tokens per query.  The visible-pair
    count from the oracle's selection (on a sample of rows, every query sees
    exactly k*B keys) reproduces the printed numbers under the convention
    stated in the golden file."""
    g = _load("page_flop_counts.json")
    n, h, d, B, k = g["n"], g["heads"], g["d"], g["block"], g["topk"]
    rng = np.random.default_rng(20)
    rows = rng.choice(h * n, size=64, replace=False).astype(np.int64)
    nb = n // B
    s = rng.standard_normal((rows.size, nb))
    idx, _, _ = oracle.topk(s, n=n, block=B, k=k, causal=False, rows=rows)
    pairs_per_query = oracle.visible_pairs(idx, n, B, False, rows) / rows.size
    assert pairs_per_query == g["tokens_per_query_printed"]
    pairs = pairs_per_query * n * h
    coarse_pairs = n * nb * h
    sparse_mm = 4 * d * pairs + 2 * d * coarse_pairs
    dense_mm = 4 * d * n * n * h
    sparse_page = sparse_mm + 5 * pairs
    dense_page = dense_mm + 5 * n * n * h

    def sig(x, digits):
        return float(f"{x:.{digits}g}")

    assert sig(sparse_page, 3) == g["sparse_flops_printed"]
    assert sig(dense_page, 3) == g["dense_flops_printed"]
    assert round(100 * sparse_page / dense_page, 1) == g["sparse_fraction_printed_percent"]
    assert sparse_mm == pytest.approx(85.899e9, rel=1e-4)
    assert dense_mm == pytest.approx(2.199e12, rel=1e-3)


# ---------------------------------------------------------------- backward --
# oracle.attend_backward follows nishantmodi.me "sparse-attention-triton-bench",
# section "What's next" (a backward pass through the softmax-weighted sum over
# the selected blocks, FlashAttention-2's backward as the dense model), with
# the selection held fixed.

def _torch_dense_grads(q, k, v, dout, scale, causal):
    """Autograd of textbook attention in fp64 (torch CPU), per head [n, d]."""
    torch = pytest.importorskip("torch")
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    z = tq @ tk.transpose(-1, -2) * scale
    if causal:
        n = q.shape[-2]
        z = z.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
    lse = torch.logsumexp(z, dim=-1)
    o = torch.softmax(z, dim=-1) @ tv
    o.backward(torch.tensor(dout, dtype=torch.float64))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy(), lse.detach().numpy()


def _all_blocks_idx(bh, n, block, topk):
    nb = -(-n // block)
    idx = np.full((bh * n, topk), -1, np.int32)
    idx[:, :nb] = np.arange(nb, dtype=np.int32)
    return idx


@pytest.mark.parametrize("causal", [False, True])
def test_backward_equals_dense_autograd_when_every_block_is_kept(causal):
    """Every block selected (k*B >= n): the gradients are those of dense
    (causal) attention, computed here by torch autograd in fp64."""
    rng = np.random.default_rng(11)
    bh, n, d, block, scale = 2, 256, 32, 64, 0.2
    q, k, v, dout = (rng.standard_normal((bh, n, d)).astype(np.float32) for _ in range(4))
    idx = _all_blocks_idx(bh, n, block, 5)          # 4 blocks + one -1 pad
    dq, lse, dk, dv = oracle.attend_backward(q, k, v, dout, idx, block, causal, scale)
    for h in range(bh):
        gq, gk, gv, gl = _torch_dense_grads(q[h], k[h], v[h], dout[h], scale, causal)
        np.testing.assert_allclose(dq[h * n:(h + 1) * n], gq, rtol=0, atol=1e-11)
        np.testing.assert_allclose(lse[h * n:(h + 1) * n], gl, rtol=0, atol=1e-11)
        np.testing.assert_allclose(dk[h * 4:(h + 1) * 4].reshape(n, d), gk, rtol=0, atol=1e-11)
        np.testing.assert_allclose(dv[h * 4:(h + 1) * 4].reshape(n, d), gv, rtol=0, atol=1e-11)


def _random_selection(rng, bh, n, block, topk, causal):
    nb = -(-n // block)
    idx = np.full((bh * n, topk), -1, np.int32)
    for r in range(bh * n):
        qb = (r % n) // block
        cand = np.arange(qb + 1) if causal else np.arange(nb)
        kk = rng.integers(1, topk + 1)                 # some rows padded with -1
        sel = rng.choice(cand, size=min(kk, cand.size), replace=False)
        if causal and qb not in sel:
            sel[0] = qb
        idx[r, :sel.size] = np.sort(sel)
    return idx


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_finite_differences_of_the_forward(causal):
    """Sparse, padded selections: every gradient entry checked is the central
    difference of the loss sum(dout * attend(...)), where attend is the
    oracle's forward (independent code: two-pass softmax over key lists)."""
    rng = np.random.default_rng(5 + causal)
    bh, n, d, block, topk, scale = 1, 64, 8, 16, 3, 0.4
    q, k, v, dout = (rng.standard_normal((bh, n, d)).astype(np.float32) for _ in range(4))
    idx = _random_selection(rng, bh, n, block, topk, causal)
    dq, _, dk, dv = oracle.attend_backward(q, k, v, dout, idx, block, causal, scale)
    grads = {"q": dq.reshape(bh, n, d), "k": dk.reshape(bh, n, d), "v": dv.reshape(bh, n, d)}

    def loss(qq, kk, vv):
        o = oracle.attend(qq, kk, vv, idx, block, causal, scale)
        return float(np.sum(o * dout.reshape(-1, d).astype(np.float64)))

    h = 2.0 ** -9
    for name in ("q", "k", "v"):
        for _ in range(12):
            i, c = int(rng.integers(n)), int(rng.integers(d))
            args = {"q": q, "k": k, "v": v}
            plus = {a: x.copy() for a, x in args.items()}
            minus = {a: x.copy() for a, x in args.items()}
            plus[name][0, i, c] += np.float32(h)       # exact in float32 for |x| < 2^14 h
            minus[name][0, i, c] -= np.float32(h)
            step = float(plus[name][0, i, c]) - float(minus[name][0, i, c])
            fd = (loss(plus["q"], plus["k"], plus["v"]) - loss(minus["q"], minus["k"], minus["v"])) / step
            assert abs(fd - grads[name][0, i, c]) <= 1e-5 * max(1.0, abs(fd)), (name, i, c, fd,
                                                                                grads[name][0, i, c])


def test_backward_invariants():
    """For any selection: sum_j dv_j = sum_i dO_i (each row's weights sum to
    one) and sum_j dk_j = 0 (each row's ds sums to zero), per head; a zero
    incoming gradient gives zero gradients; key blocks nobody selects get 0."""
    rng = np.random.default_rng(21)
    bh, n, d, block, topk, scale = 2, 256, 16, 32, 3, 0.3
    q, k, v, dout = (rng.standard_normal((bh, n, d)).astype(np.float32) for _ in range(4))
    idx = _random_selection(rng, bh, n, block, topk, False)
    idx[idx == 7] = 6                                   # block 7 never selected (dups allowed)
    dq, lse, dk, dv = oracle.attend_backward(q, k, v, dout, idx, block, False, scale)
    nb = n // block
    for h in range(bh):
        np.testing.assert_allclose(dv[h * nb:(h + 1) * nb].reshape(n, d).sum(0),
                                   dout[h].astype(np.float64).sum(0), atol=1e-10)
        np.testing.assert_allclose(dk[h * nb:(h + 1) * nb].reshape(n, d).sum(0), 0.0, atol=1e-10)
        assert not dk[h * nb + 7].any() and not dv[h * nb + 7].any()
    z = oracle.attend_backward(q, k, v, np.zeros_like(dout), idx, block, False, scale)
    assert not z[0].any() and not z[2].any() and not z[3].any()
    np.testing.assert_array_equal(z[1], lse)


def test_backward_row_and_block_subsets_agree_with_the_full_call():
    rng = np.random.default_rng(3)
    bh, n, d, block, topk, scale = 2, 128, 16, 32, 2, 0.25
    q, k, v, dout = (rng.standard_normal((bh, n, d)).astype(np.float32) for _ in range(4))
    idx = _random_selection(rng, bh, n, block, topk, True)
    full = oracle.attend_backward(q, k, v, dout, idx, block, True, scale)
    rows = np.array([3, 130, 255])
    blocks = np.array([7, 0, 5])
    sub = oracle.attend_backward(q, k, v, dout, idx, block, True, scale, rows=rows, key_blocks=blocks)
    np.testing.assert_array_equal(sub[0], full[0][rows])
    np.testing.assert_array_equal(sub[1], full[1][rows])
    np.testing.assert_array_equal(sub[2], full[2][blocks])
    np.testing.assert_array_equal(sub[3], full[3][blocks])
