"""The adjacent steps at the full size of the batched GQA decode (B 16, Hq 64,
Hkv 8, d 128, L 131072, k 4096, bf16), in the launch configurations the bench
times, checked on sampled rows the oracle computes one by one and by
properties that hold on every row:

- certified adaptive k (eps 0.9, k_min 1, k_max 4096): on sampled rows the
  GPU's k, tau and kept positions are valid against the oracle's fp64 masses
  on the GPU's score row; on every row k lies in [1, 4096] and the list is
  ascending, in range, padded with -1; the step equals the adaptive select on
  the scores of topk_attn_score bitwise;
- two-level selection (blocks of 64, 128 blocks kept): level by level on
  sampled rows against the oracle's block means and exact scores;
- four causal queries per sequence: per-query scores within the exact-score
  bound, NaN where a query cannot see, kept positions bit-exact, outputs
  within tolerance;
- the cache append at the last position of a cache with spare capacity: rows
  bitwise in place, the last block's mean equal to a fresh build bitwise.
"""
import numpy as np
import pytest
import torch

import fixtures as fx
import oracle as orc
from tests.gpu_common import as_f64, dev, exact_score_bound, gpu_scores_np, problem, say, tka, tol
from tests.test_gpu_adaptive import check_rows

pytestmark = pytest.mark.gpu

W = fx.WORKLOADS["C3"]


@pytest.fixture(scope="module")
def c3():
    say(f"[full size next] generating {W}")
    q, K, V = fx.make_attn(W)
    data = dict(q=q, K=K, V=V, qt=dev(q), Kt=dev(K), Vt=dev(V))
    yield data
    data.clear()
    torch.cuda.empty_cache()


def sample_rows(n):
    return sorted({r for r in (0, 1, n // 3 + 1, n // 2 + 7, n - 1) if 0 <= r < n})


def check_list(idx: torch.Tensor, kk: torch.Tensor, n: int):
    """Every row r: idx[r, :kk[r]] ascending in [0, n), idx[r, kk[r]:] == -1."""
    k = idx.shape[-1]
    pos = torch.arange(k, device=idx.device)[None, :]
    head = pos < kk[:, None].long()
    assert bool(((idx == -1) | head).all())
    assert bool(((idx >= 0) & (idx < n) | ~head).all())
    inc = (idx[:, 1:] > idx[:, :-1]) | ~head[:, 1:]
    assert bool(inc.all())


def test_adaptive_full_size(c3):
    m = tka()
    w, rows = W, W.B * W.Hq
    p = problem(w)
    eps = 0.9
    say("[full size next] adaptive step")
    out, idx, k, tau = m.topk_decode_adaptive(p, c3["qt"], c3["Kt"], c3["Vt"], eps, 1)
    sc = m.topk_attn_score(p, c3["qt"], c3["Kt"]).reshape(rows, w.L)
    idx_s, k_s, tau_s, _ = m.topk_select_adaptive(sc, eps, 1, w.k)
    torch.cuda.synchronize()
    idx, k, tau = idx.reshape(rows, w.k), k.reshape(rows), tau.reshape(rows)
    assert torch.equal(idx, idx_s) and torch.equal(k, k_s) and torch.equal(tau.view(torch.int32),
                                                                              tau_s.view(torch.int32))
    assert bool((k >= 1).all()) and bool((k <= w.k).all())
    check_list(idx, k, w.L)
    assert bool(torch.isfinite(out).all())
    sel = sample_rows(rows)
    s = gpu_scores_np(sc[sel]).astype(np.float32)
    gi, gk, gt = idx[sel].cpu().numpy(), k[sel].cpu().numpy(), tau[sel].cpu().numpy()
    check_rows(s, eps, 1, w.k, gi, gk, gt)
    op = orc.problem_for(w)
    want = orc.attend(op, c3["q"], c3["K"], c3["V"], gi, list_mode=2, rows=sel)
    err = np.abs(out.reshape(rows, w.d)[sel].cpu().numpy().astype(np.float64) - want).max()
    say(f"[full size next] adaptive: k {int(k.min())}..{int(k.max())}, output error {err:.3g}")
    assert err <= tol(w)


def test_two_level_full_size(c3):
    m = tka()
    w, rows = W, W.B * W.Hq
    KB, b = 128, 64
    nb = (w.L + b - 1) // b
    ph = m.problem(m.HISA, w.B, w.Hq, w.Hkv, w.d, w.L, w.k, m.TKA_BF16, 0.0, b, top_blocks=KB)
    say("[full size next] two-level step")
    means = m.topk_block_mean_build(ph, c3["Kt"])
    out, idx, blk, bs, cs = m.topk_hisa_decode(ph, c3["qt"], c3["Kt"], c3["Vt"], means, want_parts=True)
    torch.cuda.synchronize()
    idx = idx.reshape(rows, w.k)
    check_list(idx, torch.full((rows,), w.k, dtype=torch.int32, device="cuda"), w.L)  # KB*b >= k: always full
    assert bool(torch.isfinite(out).all())
    sel = sample_rows(rows)
    bs_g = bs.reshape(rows, nb)[sel].cpu().numpy().astype(np.float64)
    blk_g = blk.reshape(rows, KB)[sel].cpu().numpy()
    cs_g = cs.reshape(rows, KB * b)[sel].cpu().numpy()
    idx_g = idx[sel].cpu().numpy()
    op = orc.problem_for(w)
    op.block = b
    mu = orc.block_means(op, c3["K"])  # [B, Hkv, nb, d] fp64
    qd = as_f64(c3["q"], w.dtype).reshape(w.B, w.Hq, w.d)
    s_ex = orc.score(orc.problem_for(w), c3["q"], c3["K"], rows=sel)
    ebound = exact_score_bound(w, c3["q"], c3["K"], sel)
    for i, r in enumerate(sel):
        bb, h = divmod(r, w.Hq)
        g = h // w.G
        # (i) block scores: an fp32 mean of b keys, then an fp32 dot product of length d
        ref = mu[bb, g] @ qd[bb, h]
        mabs = np.abs(as_f64(c3["K"][bb, g], w.dtype)).reshape(nb, b, w.d).mean(1)
        bound = mabs @ np.abs(qd[bb, h]) * (w.d + b + 2) * 2.0 ** -23 + 1e-30
        assert np.all(np.abs(bs_g[i] - ref) <= bound), r
        # (ii) kept blocks on the GPU's block scores
        assert np.array_equal(blk_g[i], orc.select(bs_g[i:i + 1].astype(np.float32), KB)[0]), r
        # (iii) candidate scores (every block is whole: L is a multiple of b)
        pos = (blk_g[i][:, None] * b + np.arange(b)[None, :]).reshape(-1)
        assert np.all(np.abs(cs_g[i] - s_ex[i, pos]) <= ebound[i, pos]), r
        # (iv) kept positions on the GPU's candidate scores
        sl = orc.select(cs_g[i:i + 1], w.k)[0]
        assert np.array_equal(idx_g[i], blk_g[i][sl // b] * b + sl % b), r
    # (v) attention over the GPU's positions
    want = orc.attend(orc.problem_for(w), c3["q"], c3["K"], c3["V"], idx_g, list_mode=2, rows=sel)
    err = np.abs(out.reshape(rows, w.d)[sel].cpu().numpy().astype(np.float64) - want).max()
    say(f"[full size next] two-level: output error {err:.3g}")
    assert err <= tol(w)


def test_four_queries_full_size(c3):
    m = tka()
    w, M = W, 4
    B, Hq, L, k, d = w.B, w.Hq, w.L, w.k, w.d
    qm = fx.encode(fx.normal(97, 0, B * M * Hq * d), fx.BF16).reshape(B, M, Hq, d)
    pm = m.problem(m.EXACT, B, Hq, w.Hkv, d, L, k, m.TKA_BF16, n_queries=M)
    qmt = dev(qm)
    say("[full size next] four queries per sequence")
    out, idx = m.topk_decode(pm, qmt, c3["Kt"], c3["Vt"])
    sc = m.topk_attn_score(pm, qmt, c3["Kt"])
    torch.cuda.synchronize()
    nr = B * M * Hq
    idx2 = idx.reshape(nr, k)
    t_of = (torch.arange(nr, device="cuda") // Hq) % M
    check_list(idx2, torch.clamp(L - M + 1 + t_of, max=k).to(torch.int32), L)
    assert bool(torch.isfinite(out).all())
    sel = sample_rows(nr) + [Hq * 2 + 3, nr - Hq - 2]  # rows of every query t
    sel = sorted(set(sel))
    S = sc.reshape(nr, L)
    gs = gpu_scores_np(S[sel])
    gi = idx2[sel].cpu().numpy()
    go = out.reshape(nr, d)[sel].cpu().numpy().astype(np.float64)
    pe = orc.problem_for(w)
    for i, r in enumerate(sel):
        bb, t, h = r // (M * Hq), (r // Hq) % M, r % Hq
        Lt = L - M + t + 1
        kk = min(k, Lt)
        q_t = np.ascontiguousarray(qm[:, t])
        row = bb * Hq + h
        ref = orc.score(pe, q_t, c3["K"], rows=[row])[0]
        Ka = np.abs(as_f64(c3["K"][bb, h // w.G], w.dtype))
        bound = Ka @ np.abs(as_f64(q_t[bb, h], w.dtype)) / np.sqrt(d) * d * 2.0 ** -23 + 1e-30
        assert np.all(np.isnan(gs[i, Lt:])), r
        assert np.all(np.abs(gs[i, :Lt] - ref[:Lt]) <= bound[:Lt]), r
        assert np.array_equal(gi[i, :kk], orc.select(np.ascontiguousarray(gs[i:i + 1, :Lt]), kk)[0]), r
        assert np.all(gi[i, kk:] == -1), r
        att = orc.attend(pe, q_t, c3["K"], c3["V"], gi[i:i + 1], list_mode=2, rows=[row])
        err = np.abs(go[i] - att[0]).max()
        assert err <= tol(w), (r, float(err))
    say(f"[full size next] four queries: {len(sel)} rows checked")


def test_append_full_size(c3):
    m = tka()
    w = W
    b, Lcap = 64, w.L
    L = Lcap  # the last position of the cache: the bench's append
    mcap = (Lcap + b - 1) // b
    ph = m.problem(m.HISA, w.B, w.Hq, w.Hkv, w.d, L, w.k, m.TKA_BF16, 0.0, b, top_blocks=128, block_capacity=mcap)
    Kt, Vt = c3["Kt"], c3["Vt"]
    means = m.topk_block_mean_build(ph, Kt)
    keep_k = Kt[:, :, L - 1].clone()
    keep_v = Vt[:, :, L - 1].clone()
    gen = torch.Generator(device="cuda").manual_seed(5)
    kn = torch.randn(keep_k.shape, generator=gen, device="cuda").to(torch.bfloat16)
    vn = torch.randn(keep_v.shape, generator=gen, device="cuda").to(torch.bfloat16)
    say("[full size next] append at the last position")
    try:
        m.topk_cache_append(ph, kn, vn, Kt, Vt, means=means)
        fresh = m.topk_block_mean_build(ph, Kt)
        torch.cuda.synchronize()
        assert torch.equal(Kt[:, :, L - 1].view(torch.int16), kn.view(torch.int16))
        assert torch.equal(Vt[:, :, L - 1].view(torch.int16), vn.view(torch.int16))
        assert torch.equal(means.view(torch.int32), fresh.view(torch.int32))
    finally:
        Kt[:, :, L - 1] = keep_k
        Vt[:, :, L - 1] = keep_v
        torch.cuda.synchronize()
