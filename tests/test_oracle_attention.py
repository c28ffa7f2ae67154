"""Pins of the oracle's scoring and attention steps.

- k = L is dense attention Attention(Q_t, K_1:t, V_1:t) ("Sparse Attention in
  LLM Inference", "The Bottleneck of Dense Attention"): checked against
  torch's scaled_dot_product_attention in fp64 on the CPU (a library routine),
  including grouped KV heads.
- Attention over an arbitrary kept set equals SDPA with a boolean mask that
  admits only that set.
- k = 1 returns the value row of the lowest-index argmax; constant value rows
  return that row.
- Exact scores: q = unit vector e_c gives scale * K[i, c]; tiny brute force in
  exact rational arithmetic.
- Block variant ("Sparse Attention Landscape", "Block Sparse Attention", MoBA
  mean-pooled keys): b = 1 reduces to unscaled token scores; tiny brute force
  of the block means with fractions.
- Indexer variant (same page, "Token Sparse Attention"): one head with weight 1
  ranks by ReLU of the dot product; all-negative dots give all-zero scores and
  the selection {0..k-1}; tiny brute force with torch's own E4M3FN decode.
"""
from fractions import Fraction

import numpy as np
import torch

import fixtures as fx
import oracle as orc


def _f32_problem(B, Hq, Hkv, d, L, k, seed=0, mode=orc.EXACT, block=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    K = rng.standard_normal((B, Hkv, L, d)).astype(np.float32)
    V = rng.standard_normal((B, Hkv, L, d)).astype(np.float32)
    p = orc.problem(mode, B, Hq, Hkv, d, L, k, orc.F32, block=block)
    return p, q, K, V


def _sdpa(q, K, V, mask=None):
    G = q.shape[1] // K.shape[1]
    qt = torch.from_numpy(q.astype(np.float64))[:, :, None, :]
    Kt = torch.from_numpy(K.astype(np.float64)).repeat_interleave(G, dim=1)
    Vt = torch.from_numpy(V.astype(np.float64)).repeat_interleave(G, dim=1)
    am = None if mask is None else torch.from_numpy(mask)[:, :, None, :]
    return torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=am)[:, :, 0, :].numpy()


def test_k_equals_L_is_dense_attention_gqa():
    p, q, K, V = _f32_problem(2, 8, 2, 64, 300, 300, seed=1)
    out, idx = orc.decode(p, q, K, V)
    assert (idx == np.arange(300)).all()
    ref = _sdpa(q, K, V).reshape(-1, 64)
    assert np.abs(out - ref).max() < 1e-12


def test_k_beyond_L_is_dense_attention():
    p, q, K, V = _f32_problem(1, 4, 4, 32, 50, 80, seed=2)
    out, idx = orc.decode(p, q, K, V)
    assert (idx[:, 50:] == -1).all()
    assert np.abs(out - _sdpa(q, K, V).reshape(-1, 32)).max() < 1e-12


def test_attend_matches_masked_sdpa():
    B, Hq, Hkv, d, L, k = 2, 4, 2, 32, 200, 37
    p, q, K, V = _f32_problem(B, Hq, Hkv, d, L, k, seed=3)
    rng = np.random.default_rng(4)
    idx = np.stack([np.sort(rng.choice(L, k, replace=False)) for _ in range(B * Hq)]).astype(np.int32)
    out = orc.attend(p, q, K, V, idx, list_mode=0)
    mask = np.zeros((B * Hq, L), bool)
    for r in range(B * Hq):
        mask[r, idx[r]] = True
    ref = _sdpa(q, K, V, mask.reshape(B, Hq, L)).reshape(-1, d)
    assert np.abs(out - ref).max() < 1e-12


def test_k1_returns_argmax_value_row():
    p, q, K, V = _f32_problem(1, 2, 1, 16, 64, 1, seed=5)
    out, idx = orc.decode(p, q, K, V)
    for h in range(2):
        s = K[0, 0].astype(np.float64) @ q[0, h].astype(np.float64)
        j = int(np.argmax(s))
        assert idx[h, 0] == j
        assert np.array_equal(out[h], V[0, 0, j].astype(np.float64))


def test_constant_value_rows():
    p, q, K, V = _f32_problem(1, 2, 2, 16, 64, 9, seed=6)
    V[:] = np.linspace(-1, 1, 16, dtype=np.float32)
    out, _ = orc.decode(p, q, K, V)
    assert np.abs(out - V[0, 0, 0].astype(np.float64)).max() < 1e-15


def test_exact_score_unit_query():
    p, q, K, V = _f32_problem(1, 3, 1, 16, 40, 4, seed=7)
    q[:] = 0
    for h, c in enumerate([0, 5, 15]):
        q[0, h, c] = 1.0
    s = orc.score(p, q, K)
    for h, c in enumerate([0, 5, 15]):
        assert np.array_equal(s[h], K[0, 0, :, c].astype(np.float64) / 4.0)  # scale 1/sqrt(16)


def test_exact_score_bruteforce_rational():
    p, q, K, V = _f32_problem(1, 2, 1, 8, 12, 3, seed=8)
    s = orc.score(p, q, K)
    for h in range(2):
        for i in range(12):
            ex = sum(Fraction(float(q[0, h, c])) * Fraction(float(K[0, 0, i, c])) for c in range(8))
            assert abs(s[h, i] - float(ex) / np.sqrt(8.0)) <= 1e-14 * (1 + abs(float(ex)))


def test_block_scores_bruteforce_and_partial_last_block():
    B, Hq, Hkv, d, L, b = 1, 2, 1, 8, 29, 4  # 8 blocks, last one holds 1 key
    p, q, K, V = _f32_problem(B, Hq, Hkv, d, L, 3, seed=9, mode=orc.BLOCK, block=b)
    s = orc.score(p, q, K)
    m = (L + b - 1) // b
    assert s.shape == (Hq, m - 1)
    for h in range(Hq):
        for j in range(m - 1):
            rows = range(j * b, min((j + 1) * b, L))
            mean = [sum(Fraction(float(K[0, 0, i, c])) for i in rows) / len(rows) for c in range(d)]
            ex = sum(Fraction(float(q[0, h, c])) * mean[c] for c in range(d))
            assert abs(s[h, j] - float(ex)) <= 1e-14 * (1 + abs(float(ex)))


def test_block_size_one_reduces_to_token_selection():
    B, Hq, Hkv, d, L, k = 1, 4, 2, 16, 90, 11
    pb, q, K, V = _f32_problem(B, Hq, Hkv, d, L, k, seed=10, mode=orc.BLOCK, block=1)
    out_b, idx_b = orc.decode(pb, q, K, V)
    pe = orc.problem(orc.EXACT, B, Hq, Hkv, d, L, k, orc.F32, scale=1.0)
    se = orc.score(pe, q, K)  # unscaled token scores
    assert np.array_equal(idx_b, orc.select(se[:, : L - 1], k))
    # attention over the kept tokens plus the current one
    tok = np.concatenate([idx_b, np.full((B * Hq, 1), L - 1, np.int32)], 1)
    pe2 = orc.problem(orc.EXACT, B, Hq, Hkv, d, L, k + 1, orc.F32)
    assert np.abs(out_b - orc.attend(pe2, q, K, V, tok, list_mode=0)).max() < 1e-13


def _indexer_inputs(B, HI, dI, L, seed):
    qI = fx.encode(np.random.default_rng(seed).standard_normal((B, HI, dI)), fx.E4M3)
    kI = fx.encode(np.random.default_rng(seed + 1).standard_normal((B, L, dI)), fx.E4M3)
    w = np.random.default_rng(seed + 2).uniform(size=(B, HI)).astype(np.float32)
    return qI, kI, w


def test_indexer_bruteforce_with_torch_e4m3():
    B, HI, dI, L = 1, 3, 8, 20
    qI, kI, w = _indexer_inputs(B, HI, dI, L, 20)
    p = orc.problem(orc.INDEXER, B, 2, 1, 8, L, 5, orc.BF16, HI=HI, dI=dI)
    s = orc.score(p, qI=qI, kI=kI, w=w)
    qd = torch.from_numpy(qI).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    kd = torch.from_numpy(kI).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for i in range(L):
        ex = sum(Fraction(float(w[0, j])) * max(Fraction(0), sum(Fraction(qd[0, j, c]) * Fraction(kd[0, i, c])
                                                                  for c in range(dI))) for j in range(HI))
        assert s[0, i] == float(ex)


def test_indexer_single_head_relu_order_and_all_negative():
    B, HI, dI, L, k = 1, 1, 16, 64, 7
    qI, kI, _ = _indexer_inputs(B, HI, dI, L, 30)
    w = np.ones((1, 1), np.float32)
    p = orc.problem(orc.INDEXER, B, 2, 1, 8, L, k, orc.BF16, HI=HI, dI=dI)
    s = orc.score(p, qI=qI, kI=kI, w=w)[0]
    dots = orc.decode_values(orc.E4M3, kI[0]) @ orc.decode_values(orc.E4M3, qI[0, 0])
    assert np.array_equal(s, np.maximum(dots, 0))
    # every dot negative: scores all zero -> positions 0..k-1
    kneg = fx.encode(-np.abs(orc.decode_values(orc.E4M3, kI)) * np.sign(orc.decode_values(orc.E4M3, qI[0, 0]))[None, None, :],
                     fx.E4M3)
    s2 = orc.score(p, qI=qI, kI=kneg, w=w)[0]
    assert (s2 == 0).all()
    assert orc.select(s2, k)[0].tolist() == list(range(k))


def test_block_means_pins():
    """Block-mean keys: b = 1 gives K itself; a block of equal keys has that key as its mean;
    the partial last block divides by its own length; <q, mean_j> is the block score."""
    w = fx.shrink(fx.WORKLOADS["C4"], 64 * 5 + 9, B=1)
    q, K, _ = fx.make_attn(w)
    p = orc.problem_for(w)
    Kd = orc.decode_values(w.dtype, K).reshape(w.B, w.Hkv, w.L, w.d)
    qd = orc.decode_values(w.dtype, q).reshape(w.B, w.Hq, w.d)
    mu = orc.block_means(p, K)
    m = mu.shape[2]
    assert m == 6
    np.testing.assert_allclose(mu[:, :, -1], Kd[:, :, 5 * 64:].sum(2) / 9, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(mu[:, :, 2], Kd[:, :, 128:192].sum(2) / 64, rtol=1e-13, atol=1e-13)
    s = orc.score(p, q, K)
    want = np.stack([mu[0, h // w.G, : m - 1] @ qd[0, h] for h in range(w.Hq)])
    np.testing.assert_allclose(s, want, rtol=1e-12, atol=1e-12)
    p.block = 1
    assert np.array_equal(orc.block_means(p, K), Kd)
    p.block = w.block
    const = np.repeat(K[:, :, :1], w.L, axis=2).copy()  # every key equal to the first
    assert np.array_equal(orc.block_means(p, const), np.repeat(Kd[:, :, :1], m, axis=2))
