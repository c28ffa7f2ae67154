"""Pins of the oracle's multi-query step (M causal queries per sequence at
positions L-M .. L-1; "Evolution of Sparse Attention in Long-Context LLMs",
section 6): M = 1 is the single-query decode; with k at least every query's
visible count it is dense causal attention, checked against torch's
scaled_dot_product_attention in fp64 on the CPU; enumeration on tiny inputs."""
import math

import numpy as np
import pytest
import torch

import fixtures as fx
import oracle as orc


def test_one_query_is_the_decode():
    w = fx.shrink(fx.WORKLOADS["C2"], 900, k=70)
    q, K, V = fx.make_attn(w)
    p = orc.problem_for(w)
    out, idx = orc.decode_mq(p, 1, q, K, V)
    ref_out, ref_idx = orc.decode(p, q, K, V)
    assert np.array_equal(idx, ref_idx)
    np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-12)


def test_large_k_is_dense_causal_attention():
    B, M, Hq, Hkv, d, L = 2, 5, 4, 2, 32, 60
    rng = np.random.default_rng(4)
    q = rng.normal(size=(B, M, Hq, d)).astype(np.float32)
    K = rng.normal(size=(B, Hkv, L, d)).astype(np.float32)
    V = rng.normal(size=(B, Hkv, L, d)).astype(np.float32)
    p = orc.problem(orc.EXACT, B, Hq, Hkv, d, L, L, fx.F32)
    out, idx = orc.decode_mq(p, M, q, K, V)
    G = Hq // Hkv
    qt = torch.from_numpy(q.astype(np.float64)).permute(0, 2, 1, 3)          # [B, Hq, M, d]
    Kt = torch.from_numpy(K.astype(np.float64)).repeat_interleave(G, dim=1)  # [B, Hq, L, d]
    Vt = torch.from_numpy(V.astype(np.float64)).repeat_interleave(G, dim=1)
    mask = torch.arange(L)[None, :] <= (L - M + torch.arange(M))[:, None]    # query t sees keys <= L-M+t
    ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mask)  # [B, Hq, M, d]
    ref = ref.permute(0, 2, 1, 3).reshape(B * M * Hq, d).numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    for r in range(B * M * Hq):
        t = (r // Hq) % M
        Lt = L - M + t + 1
        assert list(idx[r, :Lt]) == list(range(Lt)) and np.all(idx[r, Lt:] == -1)


@pytest.mark.parametrize("seed", range(5))
def test_tiny_inputs_against_enumeration(seed):
    rng = np.random.default_rng(seed)
    B, M, Hq, Hkv, d = 1, int(rng.integers(1, 4)), 2, 1, 4
    L, k = int(rng.integers(M, 12)), int(rng.integers(1, 6))
    q = rng.normal(size=(B, M, Hq, d)).astype(np.float32)
    K = rng.normal(size=(B, Hkv, L, d)).astype(np.float32)
    V = rng.normal(size=(B, Hkv, L, d)).astype(np.float32)
    if seed % 2:
        K = np.round(K).astype(np.float32)
        q = np.round(q).astype(np.float32)
    p = orc.problem(orc.EXACT, B, Hq, Hkv, d, L, k, fx.F32)
    out, idx = orc.decode_mq(p, M, q, K, V)
    for t in range(M):
        for h in range(Hq):
            r = t * Hq + h
            Lt = L - M + t + 1
            z = {i: float(q[0, t, h].astype(np.float64) @ K[0, 0, i].astype(np.float64)) / math.sqrt(d)
                 for i in range(Lt)}
            top = sorted(sorted(range(Lt), key=lambda i: (-z[i], i))[:k])
            assert list(idx[r, :len(top)]) == top and np.all(idx[r, len(top):] == -1)
            zz = np.array([z[i] for i in top])
            wgt = np.exp(zz - zz.max())
            ref = (wgt[:, None] * V[0, 0, top].astype(np.float64)).sum(0) / wgt.sum()
            np.testing.assert_allclose(out[r], ref, rtol=1e-12, atol=1e-12)
