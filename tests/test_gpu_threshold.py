"""topk_attn_score_threshold: the kept (score, position) pairs of each row are
exactly the scores of topk_attn_score that rank at or above the row's
threshold (IEEE order, -0 == +0), bit for bit, and a second call appends the
same set after the first."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import fixtures as fx
from tests.gpu_common import dev, problem, say, tka

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("L,k", [(9000, 300), (40000, 2048)])
def test_threshold_scan_keeps_exactly_the_ranked_set(L, k):
    w = fx.shrink(fx.WORKLOADS["C3"], L, B=2, k=k)
    m = tka()
    q, K, V = fx.make_attn(w)
    qt, Kt = dev(q), dev(K)
    p = problem(w)
    rows = w.B * w.Hq
    s = m.topk_attn_score(p, qt, Kt).reshape(rows, L)
    srt = torch.sort(s, dim=1, descending=True).values
    thr = srt[:, k - 1].contiguous()                 # the k-th largest score of each row
    thr[0] = srt[0, 0]                                # a row keeping only its maximum
    thr[1] = -torch.inf                               # a row keeping everything
    cap = L
    counts = torch.zeros(rows, dtype=torch.int32, device="cuda")
    cs = torch.empty((rows, cap), dtype=torch.float32, device="cuda")
    cp = torch.empty((rows, cap), dtype=torch.int32, device="cuda")
    say(f"[threshold] L={L} k={k}")
    m.topk_attn_score_threshold(p, qt, Kt, thr, counts, cs, cp)
    torch.cuda.synchronize()
    s_np, thr_np = s.cpu().numpy(), thr.cpu().numpy()
    c_np, cs_np, cp_np = counts.cpu().numpy(), cs.cpu().numpy(), cp.cpu().numpy()
    for r in range(rows):
        want = np.nonzero(s_np[r] >= thr_np[r])[0]
        assert c_np[r] == len(want), r
        got = np.sort(cp_np[r, : c_np[r]])
        assert np.array_equal(got, want), r
        order = np.argsort(cp_np[r, : c_np[r]])
        assert np.array_equal(cs_np[r, : c_np[r]][order].view(np.uint32), s_np[r, want].view(np.uint32))
    # append: the same pairs again after the first batch (rows that still fit)
    before = counts.clone()
    m.topk_attn_score_threshold(p, qt, Kt, thr, counts, cs, cp)
    torch.cuda.synchronize()
    assert torch.equal(counts, 2 * before)
    c2 = counts.cpu().numpy()
    cp2 = cp.cpu().numpy()
    for r in range(rows):
        n1 = before[r].item()
        if 2 * n1 <= cap:
            assert np.array_equal(np.sort(cp2[r, n1: 2 * n1]), np.sort(cp_np[r, :n1]))


def _check_kept(s_np, thr_np, c_np, cs_np, cp_np):
    for r in range(s_np.shape[0]):
        want = np.nonzero(s_np[r] >= thr_np[r])[0]
        assert c_np[r] == len(want), r
        order = np.argsort(cp_np[r, : c_np[r]])
        assert np.array_equal(cp_np[r, : c_np[r]][order], want), r
        assert np.array_equal(cs_np[r, : c_np[r]][order].view(np.uint32), s_np[r, want].view(np.uint32)), r


@pytest.mark.parametrize("G,d", [(2, 128), (4, 64), (16, 128), (8, 256)])
def test_threshold_scan_head_groupings(G, d):
    """The per-head stages hold fewer pairs as G and d grow; rows keeping everything overflow a
    stage on most tiles, rows keeping a third now and then, rows keeping their maximum never.
    Every row's kept set stays exact."""
    w = replace(fx.shrink(fx.WORKLOADS["C3"], 20000, B=1, Hq=2 * G, Hkv=2, k=512), d=d)
    m = tka()
    q, K, V = fx.make_attn(w)
    qt, Kt = dev(q), dev(K)
    p = problem(w)
    rows, L = w.B * w.Hq, w.L
    s = m.topk_attn_score(p, qt, Kt).reshape(rows, L)
    srt = torch.sort(s, dim=1, descending=True).values
    thr = torch.empty(rows, dtype=torch.float32, device="cuda")
    for r in range(rows):
        thr[r] = -torch.inf if r % 3 == 0 else (srt[r, L // 3] if r % 3 == 1 else srt[r, 0])
    counts = torch.zeros(rows, dtype=torch.int32, device="cuda")
    cs = torch.empty((rows, L), dtype=torch.float32, device="cuda")
    cp = torch.empty((rows, L), dtype=torch.int32, device="cuda")
    say(f"[threshold groupings] G={G} d={d}")
    m.topk_attn_score_threshold(p, qt, Kt, thr, counts, cs, cp)
    torch.cuda.synchronize()
    _check_kept(s.cpu().numpy(), thr.cpu().numpy(), counts.cpu().numpy(), cs.cpu().numpy(), cp.cpu().numpy())


@pytest.mark.parametrize("M,G,d", [(2, 8, 128), (4, 8, 128), (3, 16, 128), (2, 4, 64), (2, 8, 256), (4, 8, 64), (2, 16, 256)])
def test_threshold_scan_several_queries(M, G, d):
    """The several-query scan (one pass over K for the M * G rows of a KV group): rows keeping every
    visible position overflow their stage on every tile, rows keeping a third now and then, rows
    keeping their maximum never, and NaN thresholds keep everything a query can see. With at most 32
    rows per group each wave scores all of them (one or two 16-row blocks) on its own tiles; above
    32 the workgroup shares each tile and each wave scores a block on both halves. Every row's kept
    set is exactly its visible scores at or above the threshold, the scores bit for bit those of
    topk_attn_score."""
    B, Hkv, L = 2, 2, 20000 + 11
    Hq = G * Hkv
    m = tka()
    w = fx.Workload("mq-threshold", fx.MODE_EXACT, B, Hq, Hkv, d, L, 512, fx.BF16, 40 + M * G, fx.PLANT_ALIGN,
                    100, 0.5)
    _, K, _ = fx.make_attn(w)
    q = fx.encode(fx.normal(50 + M * G, 0, B * M * Hq * d), fx.BF16).reshape(B, M, Hq, d)
    qt, Kt = dev(q), dev(K)
    p = m.problem(m.EXACT, B, Hq, Hkv, d, L, 512, m.TKA_BF16, n_queries=M)
    rows = B * M * Hq
    s = m.topk_attn_score(p, qt, Kt).reshape(rows, L)
    s_np = s.cpu().numpy()
    thr_np = np.empty(rows, np.float32)
    for r in range(rows):
        t = (r // Hq) % M
        vis = np.sort(s_np[r, : L - M + t + 1])[::-1]
        thr_np[r] = [-np.inf, vis[len(vis) // 3], vis[0], np.nan][r % 4]
    thr = torch.from_numpy(thr_np).cuda()
    counts = torch.zeros(rows, dtype=torch.int32, device="cuda")
    cs = torch.empty((rows, L), dtype=torch.float32, device="cuda")
    cp = torch.empty((rows, L), dtype=torch.int32, device="cuda")
    say(f"[threshold several queries] M={M} G={G} d={d}")
    m.topk_attn_score_threshold(p, qt, Kt, thr, counts, cs, cp)
    torch.cuda.synchronize()
    c_np, cs_np, cp_np = counts.cpu().numpy(), cs.cpu().numpy(), cp.cpu().numpy()
    for r in range(rows):
        t = (r // Hq) % M
        vis = L - M + t + 1
        assert np.isnan(s_np[r, vis:]).all()
        want = np.arange(vis) if np.isnan(thr_np[r]) else np.nonzero(s_np[r, :vis] >= thr_np[r])[0]
        assert c_np[r] == len(want), (r, c_np[r], len(want))
        order = np.argsort(cp_np[r, : c_np[r]])
        assert np.array_equal(cp_np[r, : c_np[r]][order], want), r
        assert np.array_equal(cs_np[r, : c_np[r]][order].view(np.uint32), s_np[r, want].view(np.uint32)), r
