"""The block-mean variant's fused step selects each row's kept blocks inside
the gather (rows of at most 2048 blocks, k <= 256): a bound from the
per-thread maxima and the few scores reaching it ranked one by one (k <= 64),
else the radix select. Against the three-call composition (indices and
outputs bitwise), the oracle's select on the GPU's own block scores (indices
exact) and the oracle's attention over the kept blocks (outputs within
tolerance), on regular rows, rows with every score tied, a crowd of tied top
blocks larger than the ranked stash, k above the ranked form's 64, and short
rows."""
import numpy as np
import pytest
import torch

import fixtures as fx
import oracle as orc
from tests.gpu_common import dev, problem, say, tka, tol

pytestmark = pytest.mark.gpu

BASE = fx.shrink(fx.WORKLOADS["C4"], 64 * 2000 + 17, B=2)  # 2001 blocks: 2000 compete, the last is current


def _run(w, q, K, V):
    m = tka()
    p = problem(w)
    qt, Kt, Vt = dev(q), dev(K), dev(V)
    means = m.topk_block_mean_build(p, Kt)
    out_f, idx_f = m.topk_decode(p, qt, Kt, Vt, proxy_keys=means)
    sc = m.topk_attn_score(p, qt, means)
    rows = w.B * w.Hq
    idx, _ = m.topk_select(sc.reshape(rows, -1), w.k, want_sel=False)
    out = m.sparse_attn_gather(p, qt, Kt, Vt, idx, idx_unit=w.block)
    torch.cuda.synchronize()
    assert torch.equal(idx_f.reshape(idx.shape), idx)
    assert torch.equal(out_f.view(torch.int32), out.view(torch.int32))
    gi = idx.cpu().numpy()
    assert np.array_equal(gi, orc.select(sc.reshape(rows, -1).cpu().numpy(), w.k))
    ref = orc.attend(orc.problem_for(w), q, K, V, gi, list_mode=0, unit=w.block)
    assert np.abs(out.cpu().numpy().reshape(-1, w.d) - ref).max() <= tol(w)
    return gi


def test_block_select_regular():
    w = BASE
    q, K, V = fx.make_attn(w)
    say("[block select] 2000 competing blocks, k 16")
    _run(w, q, K, V)


def test_block_select_all_scores_tied():
    w = BASE
    q, K, V = fx.make_attn(w)
    K[:] = K[0, 0, 0]  # every block mean equal: every score of a row ties
    say("[block select] every score tied")
    gi = _run(w, q, K, V)
    assert (gi == np.arange(w.k)).all()


def test_block_select_tied_crowd_beyond_the_stash():
    """300 blocks per KV head share one high mean: the bound admits all 300 (more than the
    256 ranked one by one), so the rows take the radix select; the kept blocks are the 16
    lowest of the crowd."""
    w = BASE
    q, K, V = fx.make_attn(w)
    qf = fx.bf16_bits_to_f32(q).astype(np.float64)
    G = w.Hq // w.Hkv
    rng = np.random.default_rng(7)
    crowd = {}
    for b in range(w.B):
        for g in range(w.Hkv):
            d = qf[b, g * G:(g + 1) * G].sum(0)
            d = 6.0 * d / np.linalg.norm(d)
            blocks = np.sort(rng.choice(1999, 300, replace=False))
            crowd[(b, g)] = blocks
            for j in blocks:
                K[b, g, j * w.block:(j + 1) * w.block] = fx.encode(np.tile(d, (w.block, 1)), fx.BF16)
    say("[block select] 300 tied top blocks per KV head")
    gi = _run(w, q, K, V).reshape(w.B, w.Hq, w.k)
    for (b, g), blocks in crowd.items():
        for h in range(g * G, (g + 1) * G):
            assert (gi[b, h] == blocks[:w.k]).all()


@pytest.mark.parametrize("k", [64, 65, 200])
def test_block_select_larger_k(k):
    w = fx.shrink(fx.WORKLOADS["C4"], 64 * 1500 + 5, B=1, k=k, seed=31)
    q, K, V = fx.make_attn(w)
    say(f"[block select] 1500 blocks, k {k}")
    _run(w, q, K, V)


def test_block_select_short_rows():
    w = fx.shrink(fx.WORKLOADS["C4"], 64 * 40 + 3, B=3, k=16, seed=32)  # 40 competing blocks
    q, K, V = fx.make_attn(w)
    say("[block select] 40 competing blocks")
    _run(w, q, K, V)
