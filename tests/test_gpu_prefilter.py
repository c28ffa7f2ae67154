"""The fused exact step's candidate prefilter (sampled threshold, candidate
scan, exact select on the candidates) and its repair path (full rescore of
rows whose candidates cannot hold the answer) must give exactly what the
three-call composition gives: indices and outputs bitwise equal, indices
equal to the oracle's select on the GPU's own score array.

The repair path is forced from the inputs: all keys equal (every score ties,
far too many candidates) and high-scoring keys planted exactly where the
sampling pass looks (the threshold lands above the k-th score)."""
import numpy as np
import pytest
import torch

import fixtures as fx
import oracle as orc
from tests.gpu_common import dev, problem, say, tka, tol

pytestmark = pytest.mark.gpu

BASE = fx.Workload("prefilter-probe", fx.MODE_EXACT, 2, 8, 2, 128, 32768, 2048, fx.BF16, 11, fx.PLANT_ALIGN, 328, 0.5)


def _run_both(w, q, K, V):
    m = tka()
    qt, Kt, Vt = dev(q), dev(K), dev(V)
    p = problem(w)
    out_f, idx_f = m.topk_decode(p, qt, Kt, Vt)
    sc = m.topk_attn_score(p, qt, Kt)
    idx, sel = m.topk_select(sc.reshape(w.B * w.Hq, w.L), w.k)
    out = m.sparse_attn_gather(p, qt, Kt, Vt, idx, sel_scores=sel)
    torch.cuda.synchronize()
    assert torch.equal(idx_f.reshape(idx.shape), idx)
    assert torch.equal(out_f.view(torch.int32), out.view(torch.int32))
    s = sc.reshape(w.B * w.Hq, w.L).cpu().numpy()
    gi = idx.cpu().numpy()
    assert np.array_equal(gi, orc.select(s, w.k))
    ref = orc.attend(orc.problem_for(w), q, K, V, gi, list_mode=0)
    assert np.abs(out.cpu().numpy().reshape(-1, w.d) - ref).max() <= tol(w)
    return gi


def test_prefilter_regular_rows():
    w = BASE
    q, K, V = fx.make_attn(w)
    say("[prefilter] planted aligned keys, no repair expected")
    _run_both(w, q, K, V)


def test_prefilter_repair_all_keys_equal():
    w = BASE
    q, K, V = fx.make_attn(w)
    K[:] = K[0, 0, 0]  # every key row identical: every score of a row ties
    say("[prefilter] all keys equal")
    gi = _run_both(w, q, K, V)
    assert (gi == np.arange(w.k)).all()  # ties go to the lowest positions


@pytest.mark.parametrize("groups", ["all", "first"])
def test_prefilter_repair_threshold_too_high(groups):
    w = BASE
    q, K, V = fx.make_attn(w)
    qf = fx.bf16_bits_to_f32(q).astype(np.float64)
    G = w.Hq // w.Hkv
    pos = np.arange(w.L)
    hot = (pos % 1024) < 64  # the runs a sampling pass reads for this shape
    for b in range(w.B):
        for g in range(w.Hkv if groups == "all" else 1):
            d = qf[b, g * G:(g + 1) * G].sum(0)
            d = d / np.linalg.norm(d)
            mag = 12.0 + 0.01 * pos[hot]  # distinct, all above every other key's score
            K[b, g, hot] = fx.encode(mag[:, None] * d[None, :], fx.BF16)
    say(f"[prefilter] hot keys at sampled positions ({groups})")
    _run_both(w, q, K, V)


def test_prefilter_repair_crowded_tie_bin():
    """2500 identical top keys per KV head: the k-th score sits in a tie run
    longer than the stash, so the row goes to the full select."""
    w = BASE
    q, K, V = fx.make_attn(w)
    qf = fx.bf16_bits_to_f32(q).astype(np.float64)
    G = w.Hq // w.Hkv
    rng = np.random.default_rng(3)
    for b in range(w.B):
        for g in range(w.Hkv):
            d = qf[b, g * G:(g + 1) * G].sum(0)
            d = 8.0 * d / np.linalg.norm(d)
            pos = np.sort(rng.choice(w.L, 2500, replace=False))
            K[b, g, pos] = fx.encode(np.tile(d, (len(pos), 1)), fx.BF16)
    say("[prefilter] crowded tie bin")
    _run_both(w, q, K, V)


def test_prefilter_repair_more_groups_than_slots():
    """L = 131072, 16 heads per KV group: a repair slot holds 16 rows x L scores (8 MiB), so the
    bounded repair runs 8 slots; 12 of the 16 groups are flagged (hot keys at every sampled
    position: the threshold lands above the k-th score), so some repair workgroups take two groups
    in turn and others one; the unflagged groups keep their prefilter result."""
    w = fx.Workload("prefilter-many-repairs", fx.MODE_EXACT, 2, 128, 8, 128, 131072, 4096, fx.BF16, 12,
                    fx.PLANT_ALIGN, 655, 0.5)
    q, K, V = fx.make_attn(w)
    qf = fx.bf16_bits_to_f32(q).astype(np.float64)
    G = w.Hq // w.Hkv
    pos = np.arange(w.L)
    hot = (pos % 4096) < 64  # the runs the sampling pass reads for this shape
    flagged = 0
    for b in range(w.B):
        for g in range(w.Hkv):
            if (b * w.Hkv + g) % 4 == 3:
                continue  # left alone
            d = qf[b, g * G:(g + 1) * G].sum(0)
            d = d / np.linalg.norm(d)
            mag = 12.0 + 0.001 * pos[hot]
            K[b, g, hot] = fx.encode(mag[:, None] * d[None, :], fx.BF16)
            flagged += 1
    assert flagged == 12
    say("[prefilter] 12 of 16 groups flagged, 8 repair slots")
    _run_both(w, q, K, V)


# ---- the indexer variant on skewed indexer keys (one kept set per sequence) ----

def _run_indexer_both(w, qI, kI, wt, q, K, V):
    """Fused step vs the three calls (indexer scores -> select -> shared-list gather), bitwise; the
    indices against the oracle's select on the GPU's indexer scores; outputs against the oracle's
    attention over them."""
    m = tka()
    p = problem(w)
    qt, Kt, Vt = dev(q), dev(K), dev(V)
    qIt, kIt, wtt = dev(qI), dev(kI), dev(wt)
    out_f, idx_f = m.topk_decode(p, qt, Kt, Vt, proxy_keys=kIt, q_idx=qIt, idx_w=wtt)
    sc = m.topk_attn_score(p, qIt, kIt, idx_w=wtt)
    idx, _ = m.topk_select(sc.reshape(w.B, w.L), w.k, want_sel=False)
    out = m.sparse_attn_gather(p, qt, Kt, Vt, idx, shared=True)
    torch.cuda.synchronize()
    assert torch.equal(idx_f.reshape(idx.shape), idx)
    assert torch.equal(out_f.view(torch.int32), out.view(torch.int32))
    gi = idx.cpu().numpy()
    assert np.array_equal(gi, orc.select(sc.reshape(w.B, w.L).cpu().numpy(), w.k))
    ref = orc.attend(orc.problem_for(w), q, K, V, gi, list_mode=1)
    assert np.abs(out.cpu().numpy().reshape(-1, w.d) - ref).max() <= tol(w)
    return gi


IDX_BASE = fx.shrink(fx.WORKLOADS["C5"], 50001, B=2)


def test_indexer_regular():
    w = IDX_BASE
    qI, kI, wt = fx.make_indexer(w)
    q, K, V = fx.make_attn(w)
    say("[indexer] two sequences, split select")
    _run_indexer_both(w, qI, kI, wt, q, K, V)


def test_indexer_hot_runs():
    """Keys aligned with the weighted query heads in runs of 64 every 512 positions of the first
    sequence: 6272 scores far above the rest, more than k, concentrated in a few histogram bins."""
    w = IDX_BASE
    qI, kI, wt = fx.make_indexer(w)
    q, K, V = fx.make_attn(w)
    qd = orc.decode_values(orc.E4M3, qI[0])  # [HI, dI]
    x = (wt[0].astype(np.float64)[:, None] * qd).sum(0)
    x = 200.0 * x / np.abs(x).max()
    pos = np.arange(w.L)
    hot = (pos % 512) < 64
    kI[0, hot] = fx.encode(np.tile(x, (int(hot.sum()), 1)).astype(np.float32), fx.E4M3)
    say("[indexer] hot runs in sequence 0")
    _run_indexer_both(w, qI, kI, wt, q, K, V)


def test_indexer_all_keys_equal():
    """Every indexer key of sequence 1 equal: all its scores tie; the kept set is the first k
    positions."""
    w = IDX_BASE
    qI, kI, wt = fx.make_indexer(w)
    q, K, V = fx.make_attn(w)
    kI[1] = kI[1, 0]
    say("[indexer] all keys equal in sequence 1")
    gi = _run_indexer_both(w, qI, kI, wt, q, K, V)
    assert (gi[1] == np.arange(w.k)).all()


# ---- the indexer select over per-chunk candidates (long rows, k' <= L / 512) ----
# Chunks of 2048 positions keep their 16 first positions in the select order; a row whose chunks
# could hold more kept positions than they kept takes the full row select.

IC_BASE = fx.shrink(fx.WORKLOADS["C5"], 200003, B=2, k=256)  # 98 chunks, the last one of 1347 positions


def test_indexer_candidates_regular():
    w = IC_BASE
    qI, kI, wt = fx.make_indexer(w)
    q, K, V = fx.make_attn(w)
    say("[indexer candidates] two sequences of 200003, k 256")
    _run_indexer_both(w, qI, kI, wt, q, K, V)


def test_indexer_candidates_crowded_chunk():
    """64 high keys inside one chunk of sequence 0: that chunk holds more kept positions than its
    16 candidates, so the row takes the full select; sequence 1 keeps the candidate result."""
    w = IC_BASE
    qI, kI, wt = fx.make_indexer(w)
    q, K, V = fx.make_attn(w)
    qd = orc.decode_values(orc.E4M3, qI[0])
    x = (wt[0].astype(np.float64)[:, None] * qd).sum(0)
    x = 200.0 * x / np.abs(x).max()
    kI[0, 3 * 2048 + 100:3 * 2048 + 164] = fx.encode(np.tile(x, (64, 1)).astype(np.float32), fx.E4M3)
    say("[indexer candidates] 64 hot keys in chunk 3 of sequence 0")
    gi = _run_indexer_both(w, qI, kI, wt, q, K, V)
    assert np.isin(np.arange(3 * 2048 + 100, 3 * 2048 + 164), gi[0]).all()


def test_indexer_candidates_all_keys_equal():
    w = IC_BASE
    qI, kI, wt = fx.make_indexer(w)
    q, K, V = fx.make_attn(w)
    kI[1] = kI[1, 0]
    say("[indexer candidates] all keys equal in sequence 1")
    gi = _run_indexer_both(w, qI, kI, wt, q, K, V)
    assert (gi[1] == np.arange(w.k)).all()


def test_indexer_candidates_many_chunks():
    """601 chunks (9616 candidates: 32 a thread in the finish) over L = 601 * 2048 - 100, with 64 hot
    keys in one chunk of sequence 0 (its full row select) and sequence 1 on its candidates."""
    w = fx.shrink(fx.WORKLOADS["C5"], 601 * 2048 - 100, B=2, Hq=8, Hkv=1, k=2048, seed=23)
    qI, kI, wt = fx.make_indexer(w)
    q, K, V = fx.make_attn(w)
    qd = orc.decode_values(orc.E4M3, qI[0])
    x = (wt[0].astype(np.float64)[:, None] * qd).sum(0)
    x = 200.0 * x / np.abs(x).max()
    kI[0, 7 * 2048 + 10:7 * 2048 + 74] = fx.encode(np.tile(x, (64, 1)).astype(np.float32), fx.E4M3)
    say("[indexer candidates] L 1230748, B 2, k 2048, 64 hot keys in chunk 7 of sequence 0")
    gi = _run_indexer_both(w, qI, kI, wt, q, K, V)
    assert np.isin(np.arange(7 * 2048 + 10, 7 * 2048 + 74), gi[0]).all()


def test_indexer_candidates_short_last_chunk():
    """L = 16 * 2048 + 5: the last chunk's 5 positions are all candidates (261 in all), k 64."""
    w = fx.shrink(fx.WORKLOADS["C5"], 16 * 2048 + 5, B=3, k=64, seed=21)
    qI, kI, wt = fx.make_indexer(w)
    q, K, V = fx.make_attn(w)
    say("[indexer candidates] L 32773, B 3, k 64")
    _run_indexer_both(w, qI, kI, wt, q, K, V)


@pytest.mark.parametrize("B", [1, 4])
def test_decode_paths_agree(B):
    """topk_decode's three decode_path values on the C2 shape (32 query heads over 8 KV heads,
    L = 32768, k = 2048): with B = 1 (2^20 scores) the automatic choice takes the dense composition,
    with B = 4 (2^22) the candidate prefilter; outputs and indices are the same bits on every path."""
    m = tka()
    w = fx.shrink(fx.WORKLOADS["C2"], fx.WORKLOADS["C2"].L, B=B)
    q, K, V = fx.make_attn(w)
    qt, Kt, Vt = dev(q), dev(K), dev(V)
    got = {}
    for path in (m.TKA_PATH_AUTO, m.TKA_PATH_PREFILTER, m.TKA_PATH_DENSE):
        say(f"[decode paths] B={B} decode_path={path}")
        got[path] = m.topk_decode(problem(w, decode_path=path), qt, Kt, Vt)
    torch.cuda.synchronize()
    ref_out, ref_idx = got[m.TKA_PATH_DENSE]
    for path, (out, idx) in got.items():
        assert torch.equal(idx, ref_idx), path
        assert torch.equal(out.view(torch.int32), ref_out.view(torch.int32)), path
    auto_ws = m.topk_decode_workspace_size(problem(w, decode_path=m.TKA_PATH_AUTO))
    pre_ws = m.topk_decode_workspace_size(problem(w, decode_path=m.TKA_PATH_PREFILTER))
    dense_ws = m.topk_decode_workspace_size(problem(w, decode_path=m.TKA_PATH_DENSE))
    assert auto_ws == (dense_ws if B == 1 else pre_ws)
