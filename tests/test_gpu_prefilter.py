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
