"""GPU parity of the two-level step (topk_hisa_decode, mode TKA_SCORE_HISA)
against the fp64 oracle, level by level, on the GPU's own intermediate
arrays:

(i)   coarse block scores within the fp32 forward-error bound of the oracle's;
(ii)  kept blocks bit-exact against the oracle's select on the GPU's block
      scores;
(iii) candidate token scores within the exact-score bound, NaN exactly where
      a kept block has no token;
(iv)  kept positions bit-exact against the oracle's select (k' = min(k,
      candidate count)) on the GPU's candidate scores, mapped to positions;
(v)   outputs within 2e-3 (bf16) / 1e-5 (fp32) of the oracle's attention over
      the GPU's positions;
(vi)  end to end against the oracle's own two-level decode: kept blocks and
      tokens agree except where the oracle's scores tie within the error
      bound at a selection boundary, and rows that agree match in output.
A second call repeats bitwise.
"""
import numpy as np
import pytest
import torch

import fixtures as fx
import oracle as orc
from tests.gpu_common import as_f64, dev, exact_score_bound, say, tka, tol

pytestmark = pytest.mark.gpu

CASES = {
    "bf16-g4": (fx.Workload("hisa-bf16-g4", fx.MODE_BLOCK, 2, 8, 2, 128, 64 * 40 + 17, 200, fx.BF16, 61,
                            fx.PLANT_BLOCK, 6, 0.5, block=64), 6),
    "f32-d64-b48": (fx.Workload("hisa-f32-d64", fx.MODE_BLOCK, 1, 4, 2, 64, 48 * 30 + 5, 100, fx.F32, 62,
                                fx.PLANT_BLOCK, 4, 0.5, block=48), 5),
    "all-blocks": (fx.Workload("hisa-all", fx.MODE_BLOCK, 1, 4, 1, 128, 64 * 3 + 10, 150, fx.BF16, 63,
                               fx.PLANT_BLOCK, 1, 0.5, block=64), 9),
    "k-above-candidates": (fx.Workload("hisa-kbig", fx.MODE_BLOCK, 1, 4, 2, 128, 64 * 20, 300, fx.BF16, 64,
                                       fx.PLANT_BLOCK, 2, 0.5, block=64), 2),
    "d256-g8": (fx.Workload("hisa-d256", fx.MODE_BLOCK, 1, 16, 2, 256, 32 * 50 + 3, 120, fx.BF16, 65,
                            fx.PLANT_BLOCK, 5, 0.5, block=32), 8),
}


def block_score_bound(w, q, K, m):
    qa = np.abs(as_f64(q, w.dtype)).reshape(w.B, w.Hq, w.d)
    Ka = np.abs(as_f64(K, w.dtype)).reshape(w.B, w.Hkv, w.L, w.d)
    pad = m * w.block - w.L
    Kp = np.concatenate([Ka, np.zeros((w.B, w.Hkv, pad, w.d))], 2) if pad else Ka
    sizes = np.minimum(w.block, w.L - np.arange(m) * w.block)
    mabs = Kp.reshape(w.B, w.Hkv, m, w.block, w.d).sum(3) / sizes[None, None, :, None]
    out = np.stack([mabs[b, h // w.G] @ qa[b, h] for b in range(w.B) for h in range(w.Hq)])
    return out * (w.d + w.block + 2) * 2.0 ** -23 + 1e-30


@pytest.mark.parametrize("name", list(CASES))
def test_hisa_levels_against_oracle(name):
    w, KB = CASES[name]
    m_ = tka()
    q, K, V = fx.make_attn(w)
    qt, Kt, Vt = dev(q), dev(K), dev(V)
    dt = m_.TKA_BF16 if w.dtype == fx.BF16 else m_.TKA_F32
    p = m_.problem(m_.HISA, w.B, w.Hq, w.Hkv, w.d, w.L, w.k, dt, 0.0, w.block, top_blocks=KB)
    means = m_.topk_block_mean_build(p, Kt)
    out, idx, blk, bs, cs = m_.topk_hisa_decode(p, qt, Kt, Vt, means, want_parts=True)
    out2, idx2 = m_.topk_hisa_decode(p, qt, Kt, Vt, means)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), out2.view(torch.int32)) and torch.equal(idx, idx2)
    rows, b, L = w.B * w.Hq, w.block, w.L
    m = (L + b - 1) // b
    bs_g = bs.cpu().numpy().reshape(rows, m)
    blk_g = blk.cpu().numpy().reshape(rows, KB)
    cs_g = cs.cpu().numpy().reshape(rows, KB * b)
    idx_g = idx.cpu().numpy().reshape(rows, w.k)
    out_g = out.cpu().numpy().reshape(rows, w.d).astype(np.float64)
    op = orc.problem_for(w)
    o_out, o_idx, o_blk, o_bs = orc.hisa_decode(op, KB, q, K, V)
    # (i) coarse scores
    bbound = block_score_bound(w, q, K, m)
    assert np.all(np.abs(bs_g - o_bs) <= bbound), float((np.abs(bs_g - o_bs) / bbound).max())
    # (ii) kept blocks on the GPU's block scores
    assert np.array_equal(blk_g, orc.select(bs_g.astype(np.float32), KB))
    # (iii) candidate scores
    pe = orc.problem_for(w)
    pe.mode = orc.EXACT
    s_ex = orc.score(pe, q, K)
    ebound = exact_score_bound(w, q, K, range(rows))
    counts = np.zeros(rows, np.int64)
    for r in range(rows):
        for j in range(KB):
            slots = cs_g[r, j * b:(j + 1) * b]
            bj = blk_g[r, j]
            n = 0 if bj < 0 else min(b, L - bj * b)
            assert np.all(np.isnan(slots[n:])), (r, j)
            if n:
                pos = np.arange(bj * b, bj * b + n)
                assert np.all(np.abs(slots[:n] - s_ex[r, pos]) <= ebound[r, pos]), (r, j)
            counts[r] += n
    # (iv) kept positions on the GPU's candidate scores
    for r in range(rows):
        kr = int(min(w.k, counts[r]))
        sl = orc.select(cs_g[r:r + 1], kr)[0]
        pos = blk_g[r, sl // b] * b + sl % b
        assert np.array_equal(idx_g[r, :kr], pos), r
        assert np.all(idx_g[r, kr:] == -1), r
    # (v) attention over the GPU's positions
    ref = orc.attend(op, q, K, V, idx_g, list_mode=0)
    assert np.abs(out_g - ref).max() <= tol(w), float(np.abs(out_g - ref).max())
    # (vi) end to end
    same_blk = np.all(blk_g == o_blk, axis=1)
    same_idx = np.all(idx_g == o_idx, axis=1)
    for r in np.nonzero(~same_blk)[0]:
        srt = np.sort(o_bs[r])[::-1]
        edge = srt[min(KB, m) - 1]
        diff = set(blk_g[r][blk_g[r] >= 0].tolist()) ^ set(o_blk[r][o_blk[r] >= 0].tolist())
        assert all(abs(o_bs[r][j] - edge) <= 2 * bbound[r].max() for j in diff), (name, r, sorted(diff))
    for r in np.nonzero(same_blk & ~same_idx)[0]:
        kr = int(min(w.k, counts[r]))
        cand_pos = [bj * b + i for bj in o_blk[r] if bj >= 0 for i in range(min(b, L - bj * b))]
        vals = np.sort(s_ex[r, cand_pos])[::-1]
        edge = vals[kr - 1]
        diff = set(idx_g[r][idx_g[r] >= 0].tolist()) ^ set(o_idx[r][o_idx[r] >= 0].tolist())
        assert all(abs(s_ex[r, i] - edge) <= 2 * ebound[r].max() for i in diff), (name, r, sorted(diff)[:6])
    agree = same_blk & same_idx
    if agree.any():
        assert np.abs(out_g[agree] - o_out[agree]).max() <= tol(w)
    say(f"[hisa] {name}: {int(agree.sum())}/{rows} rows identical end to end, "
        f"candidates per row {counts.min()}..{counts.max()}")
