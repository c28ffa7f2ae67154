"""GPU parity of several causal queries per sequence (tka_problem.n_queries =
M > 1: query t at position L-M+t sees keys 0 .. L-M+t and keeps
k' = min(k, L-M+t+1) of them) against the fp64 oracle.

Scores: within the exact-score bound of the oracle's per-query scores, NaN
exactly where a query cannot see. Kept positions: bit-exact against the
oracle's select (k' per query) on the GPU's scores. Outputs: within the
tolerance of the oracle's attention over the GPU's positions, end to end
against the oracle's own multi-query decode except at near-ties, the fused
step equal to score -> select -> gather bitwise, a second call bitwise equal.
"""
import numpy as np
import pytest
import torch

import fixtures as fx
import oracle as orc
from tests.gpu_common import dev, exact_score_bound, say, tka, tol

pytestmark = pytest.mark.gpu

# name: (B, M, Hq, Hkv, d, L, k); from L = 8192 (and M <= 4, k <= L/8) the fused step takes the
# candidate prefilter (sampled thresholds, one scan of K for all M queries, exact select on the
# candidates), which must give what the dense composition gives, bitwise
CASES = {
    "g4-m4": (2, 4, 8, 2, 128, 3000, 256),
    "g8-m8": (1, 8, 16, 2, 128, 5000, 512),
    "g1-m3": (2, 3, 4, 4, 64, 1000, 100),
    "k-above-visible": (1, 5, 4, 1, 128, 300, 298),
    "d256-m2": (1, 2, 16, 2, 256, 2000, 128),
    "prefilter-g8-m4": (2, 4, 16, 2, 128, 16384, 512),
    "prefilter-g16-m3": (1, 3, 32, 2, 128, 12000, 700),
    "prefilter-g4-m2-d64": (2, 2, 8, 2, 64, 8192, 1024),
    "prefilter-g8-m3": (1, 3, 16, 2, 128, 16384, 1024),  # 24 rows: the second 16-row block half full
    "prefilter-g2-m2": (2, 2, 8, 4, 128, 8192, 256),     # 4 rows in one block
    "prefilter-g8-m2-d256": (1, 2, 16, 2, 256, 8192, 512),
    "prefilter-g16-m2": (1, 2, 32, 2, 128, 12000, 700),  # 32 rows: two full blocks, 16 heads a query
    "prefilter-g8-m4-d64": (1, 4, 16, 2, 64, 9000, 512),
}


def make(name):
    B, M, Hq, Hkv, d, L, k = CASES[name]
    w = fx.Workload("mq-" + name, fx.MODE_EXACT, B, Hq, Hkv, d, L, k, fx.BF16, 71 + len(name), fx.PLANT_ALIGN,
                    max(1, L // 200), 0.5)
    _, K, V = fx.make_attn(w)
    q = fx.encode(fx.normal(90 + len(name), 0, B * M * Hq * d), fx.BF16).reshape(B, M, Hq, d)
    return w, M, q, K, V


@pytest.mark.parametrize("name", list(CASES))
def test_several_queries_against_oracle(name):
    w, M, q, K, V = make(name)
    check_several_queries(name, w, M, q, K, V)


def test_prefilter_repair_several_queries():
    """Keys far above the rest planted exactly at the sampled positions of the first KV group of
    each sequence (positions with p % 512 < 64 for L = 16384, k = 512): the sampled threshold of
    its rows lands above their k-th score, so those rows take the full rescore and select."""
    w, M, q, K, V = make("prefilter-g8-m4")
    qf = fx.bf16_bits_to_f32(q).astype(np.float64)
    pos = np.arange(w.L)
    hot = (pos % 512) < 64
    for b in range(w.B):
        d = qf[b, :, :w.G].reshape(-1, w.d).sum(0)
        d = d / np.linalg.norm(d)
        mag = 12.0 + 0.01 * pos[hot]
        K[b, 0, hot] = fx.encode(mag[:, None] * d[None, :], fx.BF16)
    check_several_queries("prefilter-hot", w, M, q, K, V)


def check_several_queries(name, w, M, q, K, V):
    m = tka()
    p = m.problem(m.EXACT, w.B, w.Hq, w.Hkv, w.d, w.L, w.k, m.TKA_BF16, n_queries=M, decode_path=m.TKA_PATH_PREFILTER)
    qt, Kt, Vt = dev(q), dev(K), dev(V)
    out, idx = m.topk_decode(p, qt, Kt, Vt)
    out2, idx2 = m.topk_decode(p, qt, Kt, Vt)
    st = m.topk_attn_score(p, qt, Kt)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), out2.view(torch.int32)) and torch.equal(idx, idx2)
    B, Hq, L, k = w.B, w.Hq, w.L, w.k
    s = st.cpu().numpy().reshape(B, M, Hq, L)
    gi = idx.cpu().numpy().reshape(B, M, Hq, k)
    go = out.cpu().numpy().reshape(B, M, Hq, w.d).astype(np.float64)
    pe = orc.problem_for(w)
    for t in range(M):
        Lt = L - M + t + 1
        kk = min(k, Lt)
        qt_np = np.ascontiguousarray(q[:, t])
        ref = orc.score(pe, qt_np, K).reshape(B, Hq, L)
        bound = exact_score_bound(w, qt_np, K, range(B * Hq)).reshape(B, Hq, L)
        st_t = s[:, t]
        assert np.all(np.isnan(st_t[:, :, Lt:])), t
        assert np.all(np.abs(st_t[:, :, :Lt] - ref[:, :, :Lt]) <= bound[:, :, :Lt]), t
        rows = st_t.reshape(B * Hq, L)
        want = orc.select(np.ascontiguousarray(rows[:, :Lt]), kk)
        got = gi[:, t].reshape(B * Hq, k)
        assert np.array_equal(got[:, :kk], want), t
        assert np.all(got[:, kk:] == -1), t
        att = orc.attend(pe, qt_np, K, V, got, list_mode=0)
        err = np.abs(go[:, t].reshape(B * Hq, w.d) - att).max()
        assert err <= tol(w), (t, float(err))
    # end to end against the oracle's own selection
    o_out, o_idx = orc.decode_mq(pe, M, q, K, V)
    gi2 = gi.reshape(-1, k)
    same = np.all(gi2 == o_idx, axis=1)
    for r in np.nonzero(~same)[0]:
        b, t, h = r // (M * Hq), (r // Hq) % M, r % Hq
        Lt = L - M + t + 1
        z = orc.score(pe, np.ascontiguousarray(q[:, t]), K).reshape(B, Hq, L)[b, h, :Lt]
        bnd = exact_score_bound(w, np.ascontiguousarray(q[:, t]), K, [b * Hq + h])[0, :Lt]
        edge = np.sort(z)[::-1][min(k, Lt) - 1]
        diff = set(gi2[r][gi2[r] >= 0].tolist()) ^ set(o_idx[r][o_idx[r] >= 0].tolist())
        assert all(abs(z[i] - edge) <= 2 * bnd.max() for i in diff), (name, r, sorted(diff)[:6])
    if same.any():
        assert np.abs(go.reshape(-1, w.d)[same] - o_out[same]).max() <= tol(w)
    # the three calls: scores, a select per query (k' keys), the gather over the lists
    sel_idx = torch.full((B, M, Hq, k), -1, dtype=torch.int32, device="cuda")
    sel_val = torch.full((B, M, Hq, k), float("-inf"), dtype=torch.float32, device="cuda")
    for t in range(M):
        Lt = L - M + t + 1
        kk = min(k, Lt)
        i_t, v_t = m.topk_select(st[:, t].reshape(B * Hq, L), kk, row_len=Lt, row_stride=L)
        sel_idx[:, t, :, :kk] = i_t.reshape(B, Hq, kk)
        sel_val[:, t, :, :kk] = v_t.reshape(B, Hq, kk)
    co = m.sparse_attn_gather(p, qt, Kt, Vt, sel_idx, sel_scores=sel_val)
    torch.cuda.synchronize()
    assert torch.equal(sel_idx, idx)
    assert torch.equal(co.view(torch.int32), out.view(torch.int32))
    say(f"[mq] {name}: {int(same.sum())}/{len(same)} rows identical end to end")
