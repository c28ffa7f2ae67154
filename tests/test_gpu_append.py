"""GPU parity of the cache-append step (topk_cache_append).

- Key/value rows appended one step at a time land bitwise where they belong
  in strided caches sized for the longest sequence.
- Block-mean keys kept current step by step (the block of each new position
  recomputed) equal a fresh topk_block_mean_build of the same cache bitwise,
  at every length, including block boundaries, and the oracle's fp64 means
  within the fp32 summation bound; a block-variant decode on the kept means
  equals one on freshly built means bitwise.
- Indexer keys appended as OCP E4M3FN codes equal the oracle's encoder bit
  for bit (ties, saturation, subnormals, NaN, signed zero), and indexer
  scores and the indexer decode read a buffer with a capacity beyond L.
"""
import numpy as np
import pytest
import torch

import fixtures as fx
import oracle as orc
from tests.gpu_common import as_f64, dev, say, tka

pytestmark = pytest.mark.gpu


def strided_problem(m, w, L, Lcap, **kw):
    return m.problem(w.mode, w.B, w.Hq, w.Hkv, w.d, L, w.k, m.TKA_BF16 if w.dtype == fx.BF16 else m.TKA_F32, 0.0,
                     w.block, w.HI, w.dI, strides=(w.Hkv * Lcap * w.d, Lcap * w.d, w.d), **kw)


@pytest.mark.parametrize("dtype", [fx.BF16, fx.F32])
def test_append_rows_and_block_means(dtype):
    m = tka()
    Lcap, L0, b = 64 * 6 + 5, 64 * 2 + 3, 64
    w = fx.Workload("append-block", fx.MODE_BLOCK, 2, 8, 4, 128, Lcap, 3, dtype, 51, fx.PLANT_BLOCK, 3, 0.5,
                    block=b)
    q, K, V = fx.make_attn(w)
    mcap = (Lcap + b - 1) // b
    to = (lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()) if dtype == fx.BF16 else \
        (lambda a: torch.from_numpy(a).cuda())
    Kfull, Vfull = to(K), to(V)
    Kc, Vc = torch.zeros_like(Kfull), torch.zeros_like(Vfull)
    Kc[:, :, :L0] = Kfull[:, :, :L0]
    Vc[:, :, :L0] = Vfull[:, :, :L0]
    means = torch.full((w.B, w.Hkv, mcap, w.d), float("nan"), dtype=torch.float32, device="cuda")
    m.topk_block_mean_build(strided_problem(m, w, L0, Lcap, block_capacity=mcap), Kc, means)
    checked = 0
    for L in range(L0 + 1, Lcap + 1):
        p = strided_problem(m, w, L, Lcap, block_capacity=mcap)
        kn = Kfull[:, :, L - 1].contiguous()
        vn = Vfull[:, :, L - 1].contiguous()
        m.topk_cache_append(p, kn, vn, Kc, Vc, means=means)
        if L % 17 == 0 or L % b in (0, 1) or L == Lcap:
            ref = torch.full_like(means, float("nan"))
            m.topk_block_mean_build(p, Kc, ref)
            nb = (L + b - 1) // b
            torch.cuda.synchronize()
            assert torch.equal(means[:, :, :nb].view(torch.int32), ref[:, :, :nb].view(torch.int32)), L
            checked += 1
    assert torch.equal(Kc.view(torch.int16 if dtype == fx.BF16 else torch.int32),
                       Kfull.view(torch.int16 if dtype == fx.BF16 else torch.int32))
    assert torch.equal(Vc.view(torch.int16 if dtype == fx.BF16 else torch.int32),
                       Vfull.view(torch.int16 if dtype == fx.BF16 else torch.int32))
    # the kept means against the oracle's fp64 means (sums of at most b terms, then a division)
    op = orc.problem_for(w)
    mu = orc.block_means(op, K)
    got = means.cpu().numpy().astype(np.float64)
    Ka = np.abs(as_f64(K, dtype)).reshape(w.B, w.Hkv, Lcap, w.d)
    pad = mcap * b - Lcap
    Kp = np.concatenate([Ka, np.zeros((w.B, w.Hkv, pad, w.d))], 2)
    sizes = np.minimum(b, Lcap - np.arange(mcap) * b)
    bound = Kp.reshape(w.B, w.Hkv, mcap, b, w.d).sum(3) / sizes[None, None, :, None] * (b + 2) * 2.0 ** -24 + 1e-30
    assert np.all(np.abs(got - mu) <= bound)
    # a decode on the kept means equals one on freshly built means, bitwise
    p = strided_problem(m, w, Lcap, Lcap, block_capacity=mcap)
    qt = to(q)
    fresh = m.topk_block_mean_build(p, Kc)
    o1, i1 = m.topk_decode(p, qt, Kc, Vc, proxy_keys=means)
    o2, i2 = m.topk_decode(p, qt, Kc, Vc, proxy_keys=fresh)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2) and torch.equal(o1.view(torch.int32), o2.view(torch.int32))
    say(f"[append] dtype={dtype}: {Lcap - L0} appends, {checked} block-mean checks")


def test_append_indexer_keys_encode_like_the_oracle():
    m = tka()
    B, dI, Lcap, L0 = 3, 64, 40, 10
    codes = np.arange(256, dtype=np.uint8)
    vals = orc.decode_values(fx.E4M3, codes)
    fin = np.sort(np.unique(vals[np.isfinite(vals)]))
    mids = ((fin[:-1] + fin[1:]) / 2).astype(np.float32)          # ties between neighbours
    rng = np.random.default_rng(9)
    battery = np.concatenate([
        fin.astype(np.float32), mids, -mids, np.nextafter(mids, np.float32(np.inf)),
        np.array([448, 449, 463.99, 464, 1e9, np.inf, -np.inf, np.nan, 0.0, -0.0, 2 ** -10, 2 ** -12, 1e-30],
                 np.float32),
        (rng.normal(size=4000) * rng.choice([1e-3, 0.1, 3, 100], 4000)).astype(np.float32)])
    n_steps = Lcap - L0
    need = n_steps * B * dI
    battery = np.resize(battery, need).reshape(n_steps, B, dI)
    kI = torch.zeros((B, Lcap + 7, dI), dtype=torch.uint8, device="cuda")  # capacity beyond the last length
    for s in range(n_steps):
        L = L0 + s + 1
        p = m.problem(m.INDEXER, B, 8, 2, 64, L, 8, m.TKA_BF16, 0.0, 0, 4, dI, idx_capacity=Lcap + 7)
        m.topk_cache_append(p, kI_new=torch.from_numpy(battery[s].copy()).cuda(), kI_cache=kI)
    torch.cuda.synchronize()
    got = kI.cpu().numpy()
    want = orc.encode_e4m3(battery)  # [steps, B, dI]
    assert np.array_equal(got[:, L0:Lcap].transpose(1, 0, 2), want)
    assert np.all(got[:, :L0] == 0) and np.all(got[:, Lcap:] == 0)


def test_indexer_scores_and_decode_with_key_capacity():
    m = tka()
    w = fx.shrink(fx.WORKLOADS["C5"], 3001, k=300)
    q, K, V = fx.make_attn(w)
    qI, kI, wt = fx.make_indexer(w)
    cap = w.L + 37
    kI_big = np.zeros((w.B, cap, w.dI), np.uint8)
    kI_big[:, :w.L] = kI.reshape(w.B, w.L, w.dI)
    p_plain = m.problem(m.INDEXER, w.B, w.Hq, w.Hkv, w.d, w.L, w.k, m.TKA_BF16, 0.0, 0, w.HI, w.dI)
    p_cap = m.problem(m.INDEXER, w.B, w.Hq, w.Hkv, w.d, w.L, w.k, m.TKA_BF16, 0.0, 0, w.HI, w.dI, idx_capacity=cap)
    qIt, wtt = dev(qI), dev(wt)
    s1 = m.topk_attn_score(p_plain, qIt, dev(kI), idx_w=wtt)
    s2 = m.topk_attn_score(p_cap, qIt, dev(kI_big), idx_w=wtt)
    qt, Kt, Vt = dev(q), dev(K), dev(V)
    o1, i1 = m.topk_decode(p_plain, qt, Kt, Vt, proxy_keys=dev(kI), q_idx=qIt, idx_w=wtt)
    o2, i2 = m.topk_decode(p_cap, qt, Kt, Vt, proxy_keys=dev(kI_big), q_idx=qIt, idx_w=wtt)
    torch.cuda.synchronize()
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))
    assert torch.equal(i1, i2) and torch.equal(o1.view(torch.int32), o2.view(torch.int32))
