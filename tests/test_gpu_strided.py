"""Every variant on strided KV caches, against the fp64 oracle.

A growing decode cache is laid out for its longest sequence, so its capacity
per (b, KV head) exceeds the current length L, and rows may be padded ("Sparse
Attention in LLM Inference", "Changes in Caching Strategy": the cache is read
in segments through a position index). Here K and V are [B, Hkv, Lcap, d + pad]
buffers holding the workload's rows in [:, :, :L, :d]; every other element is
NaN (bf16 0x7fc0, fp32 NaN), so a kernel that reads a padding column or a
position at or beyond L turns an output or a score into NaN. The oracle reads
the same buffers through the same element strides.

Bars (as in the contiguous parity tests): scores within the fp32
forward-error bound; indices bit-exact against the oracle's select on the
GPU's own score array; outputs within 2e-3 (bf16) / 1e-5 (fp32) of the
oracle's attention over the GPU's index set; fused == three calls bitwise."""
import numpy as np
import pytest
import torch

import fixtures as fx
import oracle as orc
from tests.gpu_common import (block_score_bound, dev, exact_score_bound, gpu_scores_np, indexer_score_bound, say,
                              tka, tol)

pytestmark = pytest.mark.gpu

BF16_NAN = np.uint16(0x7FC0)


def padded(X: np.ndarray, Lcap: int, pad: int) -> np.ndarray:
    """[B, Hkv, L, d] -> [B, Hkv, Lcap, d + pad], NaN outside the workload's rows."""
    B, H, L, d = X.shape
    fill = BF16_NAN if X.dtype == np.uint16 else np.float32(np.nan)
    out = np.full((B, H, Lcap, d + pad), fill, X.dtype)
    out[:, :, :L, :d] = X
    return out


def strides_of(Xs: np.ndarray):
    _, H, Lcap, row = Xs.shape
    return (H * Lcap * row, Lcap * row, row)


def gpu_problem(w, strides, **kw):
    m = tka()
    dt = m.TKA_BF16 if w.dtype == fx.BF16 else m.TKA_F32
    kw.setdefault("decode_path", m.TKA_PATH_PREFILTER)  # the prefilter wherever it applies, as at full size
    return m.problem(w.mode, w.B, w.Hq, w.Hkv, w.d, w.L, w.k, dt, 0.0, w.block, w.HI, w.dI, strides=strides, **kw)


def oracle_problem(w, strides):
    return orc.problem(w.mode, w.B, w.Hq, w.Hkv, w.d, w.L, w.k, w.dtype, 0.0, w.block, w.HI, w.dI,
                       strides=strides)


class Case:
    def __init__(self, w, Lcap, pad):
        self.w = w
        self.q, K, V = fx.make_attn(w)
        self.K0 = K  # contiguous copy for the error bound
        self.Ks, self.Vs = padded(K, Lcap, pad), padded(V, Lcap, pad)
        self.strides = strides_of(self.Ks)
        self.qt, self.Kt, self.Vt = dev(self.q), dev(self.Ks), dev(self.Vs)
        self.p = gpu_problem(w, self.strides)
        self.op = oracle_problem(w, self.strides)


def _index_props(gi, k, n):
    kk = min(k, n)
    assert (gi[:, kk:] == -1).all()
    assert (gi[:, :kk] >= 0).all() and (gi[:, :kk] < n).all()
    if kk > 1:
        assert (np.diff(gi[:, :kk], axis=1) > 0).all()


EXACT_CASES = {
    # fused step through the candidate prefilter (bf16, G = 8, k' <= L/8, L >= 8192), ragged L
    "prefilter-g8": (fx.Workload("strided-exact-g8", fx.MODE_EXACT, 2, 16, 2, 128, 16384 + 37, 1024, fx.BF16, 31,
                                 fx.PLANT_ALIGN, 82, 0.5), 16384 + 37 + 3000, 8),
    # no prefilter (k' > L/8): full scores, row select, gather
    "dense-g4": (fx.Workload("strided-exact-g4", fx.MODE_EXACT, 2, 8, 2, 128, 5003, 1000, fx.BF16, 32,
                             fx.PLANT_ALIGN, 50, 0.5), 6000, 8),
    # head dim 64, G = 16, capacity only (no row padding)
    "prefilter-d64-g16": (fx.Workload("strided-exact-d64", fx.MODE_EXACT, 1, 16, 1, 64, 9001, 512, fx.BF16, 33,
                                      fx.PLANT_ALIGN, 90, 0.5), 12000, 0),
    # fp32 caches (vector scorer), rows padded by 4 floats
    "f32-g4": (fx.Workload("strided-exact-f32", fx.MODE_EXACT, 1, 8, 2, 64, 3001, 128, fx.F32, 34,
                           fx.PLANT_SCALE, 16, 3.0), 4000, 4),
}


@pytest.mark.parametrize("name", list(EXACT_CASES))
def test_exact_strided(name):
    w, Lcap, pad = EXACT_CASES[name]
    m = tka()
    say(f"[strided] {name}: {w}, Lcap {Lcap}, row pad {pad}")
    c = Case(w, Lcap, pad)
    rows = w.B * w.Hq
    sc = m.topk_attn_score(c.p, c.qt, c.Kt)
    s = gpu_scores_np(sc).reshape(rows, w.L)
    ref = orc.score(c.op, c.q, c.Ks)
    bound = exact_score_bound(w, c.q, c.K0, range(rows))
    assert np.all(np.abs(s - ref) <= bound), float((np.abs(s - ref) / bound).max())
    idx, sel = m.topk_select(sc.reshape(rows, w.L), w.k)
    out3 = m.sparse_attn_gather(c.p, c.qt, c.Kt, c.Vt, idx, sel_scores=sel)
    out_k = m.sparse_attn_gather(c.p, c.qt, c.Kt, c.Vt, idx)  # logits re-read from the K rows
    out_f, idx_f = m.topk_decode(c.p, c.qt, c.Kt, c.Vt)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    _index_props(gi, w.k, w.L)
    assert np.array_equal(gi, orc.select(s, w.k))
    assert torch.equal(idx_f.reshape(idx.shape), idx)
    assert torch.equal(out_f.view(torch.int32), out3.view(torch.int32))
    want = orc.attend(c.op, c.q, c.Ks, c.Vs, gi, list_mode=0)
    for got in (out3, out_k):
        err = float(np.abs(got.cpu().numpy().reshape(-1, w.d) - want).max())
        assert err <= tol(w), err
    say(f"[strided] {name}: ok")


def test_block_mean_strided():
    """Block means built from a strided K, block scores, select, gather over block runs of the strided K/V."""
    w = fx.shrink(fx.WORKLOADS["C4"], 64 * 150 + 17, B=2)
    m = tka()
    Lcap, pad = w.L + 700, 8
    say(f"[strided] block mean: {w}, Lcap {Lcap}")
    c = Case(w, Lcap, pad)
    mcap = (Lcap + w.block - 1) // w.block
    p = gpu_problem(w, c.strides, block_capacity=mcap)
    means = m.topk_block_mean_build(p, c.Kt)
    mt = (w.L + w.block - 1) // w.block
    gm = means[:, :, :mt].cpu().numpy().astype(np.float64)
    om = orc.block_means(c.op, c.Ks)
    assert np.abs(gm - om).max() <= 1e-5 * max(1.0, float(np.abs(om).max()))
    sc = m.topk_attn_score(p, c.qt, means)
    rows, n = w.B * w.Hq, mt - 1
    s = gpu_scores_np(sc).reshape(rows, n)
    ref = orc.score(c.op, c.q, c.Ks)
    bound = block_score_bound(w, c.q, c.K0)
    assert np.all(np.abs(s - ref) <= bound), float((np.abs(s - ref) / bound).max())
    idx, _ = m.topk_select(sc.reshape(rows, n), w.k, want_sel=False)
    out3 = m.sparse_attn_gather(p, c.qt, c.Kt, c.Vt, idx, idx_unit=w.block)
    out_f, idx_f = m.topk_decode(p, c.qt, c.Kt, c.Vt, proxy_keys=means)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    _index_props(gi, w.k, n)
    assert np.array_equal(gi, orc.select(s, w.k))
    assert torch.equal(idx_f.reshape(idx.shape), idx)
    assert torch.equal(out_f.view(torch.int32), out3.view(torch.int32))
    want = orc.attend(c.op, c.q, c.Ks, c.Vs, gi, unit=w.block, list_mode=0)
    err = float(np.abs(out3.cpu().numpy().reshape(-1, w.d) - want).max())
    assert err <= tol(w), err


def test_indexer_strided():
    """Indexer keys in a buffer with capacity beyond L (its tail holds the largest E4M3 code, so a read past L
    would win the selection), shared kept set, gather over the strided K/V."""
    w = fx.shrink(fx.WORKLOADS["C5"], 50001)
    m = tka()
    Lcap, pad = w.L + 999, 8
    say(f"[strided] indexer: {w}, Lcap {Lcap}")
    c = Case(w, Lcap, pad)
    qI, kI, wt = fx.make_indexer(w)
    kIc = np.full((w.B, Lcap, w.dI), 0x7E, np.uint8)
    kIc[:, : w.L] = kI
    p = gpu_problem(w, c.strides, idx_capacity=Lcap)
    qIt, kIt, wtt = dev(qI), dev(kIc), dev(wt)
    sc = m.topk_attn_score(p, qIt, kIt, idx_w=wtt)
    s = gpu_scores_np(sc).reshape(w.B, w.L)
    ref = orc.score(c.op, qI=qI, kI=kI, w=wt)
    bound = np.stack([indexer_score_bound(w, qI, kI, wt, b) for b in range(w.B)])
    assert np.all(np.abs(s - ref) <= bound)
    idx, _ = m.topk_select(sc.reshape(w.B, w.L), w.k, want_sel=False)
    out3 = m.sparse_attn_gather(p, c.qt, c.Kt, c.Vt, idx, shared=True)
    out_f, idx_f = m.topk_decode(p, c.qt, c.Kt, c.Vt, proxy_keys=kIt, q_idx=qIt, idx_w=wtt)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    _index_props(gi, w.k, w.L)
    assert np.array_equal(gi, orc.select(s, w.k))
    assert torch.equal(idx_f.reshape(idx.shape), idx)
    assert torch.equal(out_f.view(torch.int32), out3.view(torch.int32))
    want = orc.attend(c.op, c.q, c.Ks, c.Vs, gi, list_mode=1)
    err = float(np.abs(out3.cpu().numpy().reshape(-1, w.d) - want).max())
    assert err <= tol(w), err


def test_two_level_strided():
    """The two-level step reads kept blocks' tokens through the strides."""
    w = fx.Workload("strided-hisa", fx.MODE_EXACT, 2, 8, 2, 128, 64 * 100 + 5, 300, fx.BF16, 35,
                    fx.PLANT_ALIGN, 64, 0.5)
    m = tka()
    Lcap, pad = w.L + 640, 8
    c = Case(w, Lcap, pad)
    KB, bsz = 12, 64
    mcap = (Lcap + bsz - 1) // bsz
    p = m.problem(m.HISA, w.B, w.Hq, w.Hkv, w.d, w.L, w.k, m.TKA_BF16, block_size=bsz, strides=c.strides,
                  block_capacity=mcap, top_blocks=KB)
    means = m.topk_block_mean_build(p, c.Kt)
    out, idx, blk, bs, cs = m.topk_hisa_decode(p, c.qt, c.Kt, c.Vt, means, want_parts=True)
    torch.cuda.synchronize()
    op = orc.problem(orc.EXACT, w.B, w.Hq, w.Hkv, w.d, w.L, w.k, w.dtype, block=bsz, strides=c.strides)
    _, _, oblk, obs = orc.hisa_decode(op, KB, c.q, c.Ks, c.Vs)
    rows = w.B * w.Hq
    gbs = bs.cpu().numpy().reshape(rows, -1).astype(np.float64)
    assert np.abs(gbs - obs).max() <= 1e-5 * max(1.0, float(np.abs(obs).max()))
    gblk = blk.cpu().numpy().reshape(rows, KB)
    assert np.array_equal(gblk, orc.select(bs.cpu().numpy().reshape(rows, -1), KB))
    # candidate scores of the GPU's kept blocks: the exact scores of their tokens, read through the strides
    gcs = cs.cpu().numpy().reshape(rows, KB * bsz)
    ref = orc.score(op, c.q, c.Ks)
    bound = exact_score_bound(w, c.q, c.K0, range(rows))
    slot = np.arange(KB * bsz)
    for r in range(rows):
        tok = np.where(gblk[r][slot // bsz] >= 0, gblk[r][slot // bsz] * bsz + slot % bsz, -1)
        ok = (tok >= 0) & (tok < w.L)
        assert np.isnan(gcs[r][~ok]).all()
        assert np.all(np.abs(gcs[r][ok] - ref[r][tok[ok]]) <= bound[r][tok[ok]]), r
    # tokens of the GPU's kept blocks, ranked by the GPU's candidate scores
    gi = idx.cpu().numpy().reshape(rows, w.k)
    for r in range(rows):
        want = orc.select(gcs[r:r + 1], w.k)[0]
        pos = np.where(want >= 0, gblk[r][np.maximum(want, 0) // bsz] * bsz + np.maximum(want, 0) % bsz, -1)
        assert np.array_equal(gi[r], pos)
    want_out = orc.attend(op, c.q, c.Ks, c.Vs, gi, list_mode=0)
    err = float(np.abs(out.cpu().numpy().reshape(-1, w.d) - want_out).max())
    assert err <= tol(w), err


def test_several_queries_strided():
    """Two causal queries per sequence through the prefilter on a strided cache, against the oracle's
    several-query decode on the GPU's scores."""
    w = fx.Workload("strided-mq", fx.MODE_EXACT, 2, 16, 2, 128, 12000 + 3, 700, fx.BF16, 36,
                    fx.PLANT_ALIGN, 60, 0.5)
    m = tka()
    M = 2
    Lcap, pad = w.L + 1000, 8
    c = Case(w, Lcap, pad)
    q = fx.normal(w.seed, 0, w.B * M * w.Hq * w.d, fx.BF16).reshape(w.B, M, w.Hq, w.d)
    qt = dev(q)
    p = gpu_problem(w, c.strides, n_queries=M)
    sc = m.topk_attn_score(p, qt, c.Kt)
    out_f, idx_f = m.topk_decode(p, qt, c.Kt, c.Vt)
    torch.cuda.synchronize()
    rows = w.B * M * w.Hq
    s = gpu_scores_np(sc).reshape(rows, w.L)
    gi = idx_f.cpu().numpy().reshape(rows, w.k)
    for r in range(rows):
        t = (r // w.Hq) % M
        vis = w.L - M + t + 1
        assert np.isnan(s[r, vis:]).all()
        assert np.array_equal(gi[r], orc.select(s[r:r + 1, :vis], w.k)[0])
    op = oracle_problem(w, c.strides)
    # attention of every row over the GPU's kept set (list per row)
    got = out_f.cpu().numpy().reshape(rows, w.d)
    for t in range(M):
        sub = [r for r in range(rows) if (r // w.Hq) % M == t]
        qs = q[:, t]  # [B, Hq, d]: rows b*Hq + h of a one-query problem
        want = orc.attend(op, np.ascontiguousarray(qs), c.Ks, c.Vs, gi[sub], list_mode=0)
        err = float(np.abs(got[sub] - want).max())
        assert err <= tol(w), (t, err)
