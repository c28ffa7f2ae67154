"""Every workload at its full size, in the launch configuration the bench
times (one fused topk_decode call).

On every row: the fused step equals the three calls (score -> select ->
gather) bitwise, indices and outputs, compared on the GPU; the indices equal
the oracle's select run on the GPU's whole fp32 score array; k' distinct
ascending in-range indices and -1 padding. On sampled rows the oracle
computes one by one: scores within the forward-error bound and outputs within
tolerance of the oracle's attention over the GPU's index set."""
import numpy as np
import pytest
import torch

import fixtures as fx
import oracle as orc
from tests.gpu_common import (dev, exact_score_bound, gpu_scores_np, indexer_score_bound, problem, say, tka,
                              tol)

pytestmark = pytest.mark.gpu


def _check_index_properties(idx: torch.Tensor, k: int, n: int):
    kk = min(k, n)
    head, tail = idx[:, :kk], idx[:, kk:]
    assert bool((tail == -1).all())
    assert bool((head >= 0).all()) and bool((head < n).all())
    if kk > 1:
        assert bool((head[:, 1:] > head[:, :-1]).all())


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4", "C5"])
def test_full_size_workload(name):
    w = fx.WORKLOADS[name]
    m = tka()
    say(f"[full size] {name}: generating {w}")
    q, K, V = fx.make_attn(w)
    qt, Kt, Vt = dev(q), dev(K), dev(V)
    p = problem(w)
    op = orc.problem_for(w)
    kw = {}
    if w.mode == fx.MODE_BLOCK:
        kw["proxy_keys"] = m.topk_block_mean_build(p, Kt)
    if w.mode == fx.MODE_INDEXER:
        qI, kI, wt = fx.make_indexer(w)
        kw = dict(proxy_keys=dev(kI), q_idx=dev(qI), idx_w=dev(wt))
    say(f"[full size] {name}: topk_decode")
    out, idx = m.topk_decode(p, qt, Kt, Vt, **kw)
    torch.cuda.synchronize()
    n = orc.score_len(op)
    idx2 = idx.reshape(-1, w.k)
    _check_index_properties(idx2, w.k, n)
    assert bool(torch.isfinite(out).all())

    say(f"[full size] {name}: the three calls")
    if w.mode == fx.MODE_INDEXER:
        scores = m.topk_attn_score(p, kw["q_idx"], kw["proxy_keys"], idx_w=kw["idx_w"])
        rows = [0]
    elif w.mode == fx.MODE_BLOCK:
        scores = m.topk_attn_score(p, qt, kw["proxy_keys"])
        rows = sorted({r for r in (0, 1, w.Hq + 5, w.B * w.Hq - 1) if r < w.B * w.Hq})
    else:
        scores = m.topk_attn_score(p, qt, Kt)
        nr = w.B * w.Hq
        rows = sorted({r for r in (0, nr // 3 + 1, nr // 2 + 7, nr - 1) if r < nr})
    S = scores.reshape(-1, n)
    exact = w.mode == fx.MODE_EXACT
    i3, v3 = m.topk_select(S, w.k, want_sel=exact)
    o3 = m.sparse_attn_gather(p, qt, Kt, Vt, i3, idx_unit=w.block if w.mode == fx.MODE_BLOCK else 0,
                              shared=w.mode == fx.MODE_INDEXER, sel_scores=v3 if exact else None)
    torch.cuda.synchronize()
    assert torch.equal(i3, idx2), "fused and three-call indices differ"
    assert torch.equal(o3.view(torch.int32), out.view(torch.int32)), "fused and three-call outputs differ"
    say(f"[full size] {name}: oracle select on all {S.shape[0]} rows of the GPU's scores")
    s_all = gpu_scores_np(S)
    gi_all = idx2.cpu().numpy()
    want_all = orc.select(s_all, w.k)
    bad = np.nonzero(~np.all(gi_all == want_all, axis=1))[0]
    assert len(bad) == 0, f"{len(bad)} rows differ, first {bad[:8].tolist()}"

    say(f"[full size] {name}: scores for sampled rows")
    assert all(0 <= r < S.shape[0] for r in rows), rows  # checked on the host before indexing on the GPU
    gs = s_all[rows].astype(np.float64)
    gi = gi_all[rows]
    if w.mode == fx.MODE_INDEXER:
        ref = orc.score(op, qI=qI, kI=kI, w=wt, rows=rows)
        bound = np.stack([indexer_score_bound(w, qI, kI, wt, b) for b in rows])
    else:
        ref = orc.score(op, q, K, rows=rows)
        bound = exact_score_bound(w, q, K, rows) if w.mode == fx.MODE_EXACT else np.abs(ref) * 1e-5 + 1e-5
    assert np.all(np.abs(gs - ref) <= bound), float((np.abs(gs - ref) / bound).max())
    assert np.array_equal(gi, orc.select(gs.astype(np.float32), w.k))

    say(f"[full size] {name}: oracle attention on the GPU's kept sets")
    got = out.reshape(-1, w.d).cpu().numpy().astype(np.float64)
    unit = w.block if w.mode == fx.MODE_BLOCK else 0
    if w.mode == fx.MODE_INDEXER:
        heads = list(range(0, w.Hq, 7)) + [w.Hq - 1]
        want = orc.attend(op, q, K, V, gi, unit=0, list_mode=3, rows=heads)
        err = np.abs(got[heads] - want).max()
    else:
        want = orc.attend(op, q, K, V, gi, unit=unit, list_mode=2, rows=rows)
        err = np.abs(got[rows] - want).max()
    say(f"[full size] {name}: max abs output error {err:.3g}")
    assert err <= tol(w)
