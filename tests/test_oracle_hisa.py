"""Pins of the oracle's two-level selection ("Sparse Attention Landscape",
"Hierarchical Sparse Attention": top-K_B blocks by a coarse block score, then
the top-k tokens inside them by the exact score, then attention).

Checked against: the exact top-k decode when every block is kept (the
candidates are then all keys), b = 1 (blocks are single keys, so the two
levels collapse to one), K_B = 1 with k >= b (the kept set is the whole best
block), and enumeration on tiny inputs."""
import numpy as np
import pytest

import fixtures as fx
import oracle as orc


def hisa_problem(w, b, k):
    p = orc.problem_for(w)
    p.block = b
    p.k = k
    return p


def test_all_blocks_kept_is_exact_top_k():
    w = fx.shrink(fx.WORKLOADS["C2"], 1500, k=100)
    q, K, V = fx.make_attn(w)
    b = 64
    m = (w.L + b - 1) // b
    out, idx, blk, _ = orc.hisa_decode(hisa_problem(w, b, w.k), m + 3, q, K, V)
    pe = orc.problem_for(w)
    ref_out, ref_idx = orc.decode(pe, q, K, V)
    assert np.array_equal(idx, ref_idx)
    np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-12)
    assert np.all(blk[:, :m] == np.arange(m)) and np.all(blk[:, m:] == -1)


def test_single_key_blocks_collapse_to_one_level():
    w = fx.shrink(fx.WORKLOADS["C2"], 700, k=40)
    q, K, V = fx.make_attn(w)
    out, idx, blk, bs = orc.hisa_decode(hisa_problem(w, 1, w.k), 90, q, K, V)
    pe = orc.problem_for(w)
    ref_out, ref_idx = orc.decode(pe, q, K, V)
    assert np.array_equal(idx, ref_idx)
    np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-12)
    # the block scores are the unscaled exact scores
    s = orc.score(pe, q, K)
    np.testing.assert_allclose(bs * (1 / np.sqrt(w.d)), s, rtol=1e-13, atol=1e-13)


def test_one_block_keeps_the_whole_best_block():
    w = fx.shrink(fx.WORKLOADS["C4"], 64 * 7 + 10, B=1)
    q, K, V = fx.make_attn(w)
    b = w.block
    out, idx, blk, bs = orc.hisa_decode(hisa_problem(w, b, b + 5), 1, q, K, V)
    best = np.argmax(bs, axis=1)  # no ties in these data
    for r in range(idx.shape[0]):
        j = best[r]
        n = min(b, w.L - j * b)
        assert blk[r, 0] == j
        assert list(idx[r, :n]) == list(range(j * b, j * b + n)) and np.all(idx[r, n:] == -1)


@pytest.mark.parametrize("seed", range(6))
def test_tiny_inputs_against_enumeration(seed):
    rng = np.random.default_rng(seed)
    L, d, b = int(rng.integers(5, 30)), 8, int(rng.integers(1, 6))
    KB, k = int(rng.integers(1, 5)), int(rng.integers(1, 9))
    q = rng.normal(size=(1, 2, d)).astype(np.float32)
    K = rng.normal(size=(1, 1, L, d)).astype(np.float32)
    V = rng.normal(size=(1, 1, L, d)).astype(np.float32)
    if seed % 2:
        K = np.round(K).astype(np.float32)  # ties
    p = orc.problem(orc.BLOCK, 1, 2, 1, d, L, k, fx.F32, block=b)
    out, idx, blk, bs = orc.hisa_decode(p, KB, q, K, V)
    m = (L + b - 1) // b
    Kd, Vd, qd = K.astype(np.float64)[0, 0], V.astype(np.float64)[0, 0], q.astype(np.float64)[0]
    for h in range(2):
        r = np.array([qd[h] @ Kd[j * b:min((j + 1) * b, L)].mean(0) for j in range(m)])
        np.testing.assert_allclose(bs[h], r, rtol=1e-12, atol=1e-12)
        order = sorted(range(m), key=lambda j: (-bs[h][j], j))
        want_blk = sorted(order[:KB])
        assert list(blk[h, :len(want_blk)]) == want_blk and np.all(blk[h, len(want_blk):] == -1)
        cand = [i for j in want_blk for i in range(j * b, min((j + 1) * b, L))]
        s = {i: (qd[h] @ Kd[i]) / np.sqrt(d) for i in cand}
        top = sorted(sorted(cand, key=lambda i: (-s[i], i))[:k])
        assert list(idx[h, :len(top)]) == top and np.all(idx[h, len(top):] == -1)
        z = np.array([s[i] for i in top])
        pw = np.exp(z - z.max())
        np.testing.assert_allclose(out[h], (pw[:, None] * Vd[top]).sum(0) / pw.sum(), rtol=1e-12, atol=1e-12)
