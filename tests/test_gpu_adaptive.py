"""GPU parity of the certified adaptive top-k (topk_select_adaptive) and the
certified step (topk_decode_adaptive) against the fp64 oracle.

The GPU's k comes from fp32 masses summed in fixed point, the oracle's from
fp64 masses, so where a prefix's discarded mass sits within rounding of eps
the two may pick neighbouring k. What is unique is checked exactly, the rest
for validity: for the GPU's k the oracle's discarded mass is within the
budget (tau <= eps + DELTA, unless k is held at k_max or the row length), one
key fewer would break it (tau > eps - DELTA, unless k is held at k_min), the
reported tau matches the oracle's tau for that k within DELTA, and the kept
positions equal the oracle's top-k for that k bit for bit. DELTA = 1e-5
bounds the fp32 mass error (exp of fp32 differences, a few ulp each) plus
the 2^-40 fixed-point truncation summed over a row.
"""
import math

import numpy as np
import pytest
import torch

import fixtures as fx
import oracle as orc
from tests.gpu_common import dev, gpu_scores_np, problem, say, tka, tol

pytestmark = pytest.mark.gpu

DELTA = 1e-5


def check_rows(s, eps, k_min, k_max, idx, k, tau):
    s = np.ascontiguousarray(s, np.float32)
    n = s.shape[1]
    lo, hi = max(k_min, 1), min(k_max, n)
    for r in range(s.shape[0]):
        kg = int(k[r])
        assert min(lo, hi) <= kg <= hi or (n == 0 and kg == 0), (r, kg, lo, hi)
        if n == 0:
            assert np.all(idx[r] == -1)
            continue
        want = orc.select(s[r:r + 1], kg)[0]
        assert np.array_equal(idx[r, :kg], want), r
        assert np.all(idx[r, kg:] == -1), r
        _, _, t_or = orc.select_adaptive(s[r], eps, kg, kg)
        t_or = t_or[0]
        if math.isnan(t_or):
            assert math.isnan(tau[r]) and kg == min(lo, hi)
            continue
        assert abs(tau[r] - t_or) <= DELTA, (r, tau[r], t_or)
        if kg < hi:
            assert t_or <= eps + DELTA, (r, kg, t_or, eps)
        if kg > lo:
            _, _, t_less = orc.select_adaptive(s[r], eps, kg - 1, kg - 1)
            assert t_less[0] > eps - DELTA, (r, kg, t_less[0], eps)


def run_select(s_dev, eps, k_min, k_max):
    m = tka()
    idx, k, tau, sel = m.topk_select_adaptive(s_dev, eps, k_min, k_max, want_sel=True)
    idx2, k2, tau2, sel2 = m.topk_select_adaptive(s_dev, eps, k_min, k_max, want_sel=True)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(k, k2) and torch.equal(tau.view(torch.int32), tau2.view(torch.int32))
    return idx.cpu().numpy(), k.cpu().numpy(), tau.cpu().numpy(), sel.cpu().numpy()


@pytest.mark.parametrize("name,L,kmax", [("C1", 1024, 1024), ("C1", 1024, 64), ("C2", 5003, 700),
                                         ("C2", 20000, 4096), ("C3", 9000, 1024)])
@pytest.mark.parametrize("eps", [np.float32(0.01), np.float32(0.1), np.float32(0.5)])
def test_adaptive_select_on_gpu_scores(name, L, kmax, eps):
    w = fx.shrink(fx.WORKLOADS[name], L)
    if name == "C3":
        w = fx.shrink(w, L, B=1)
    q, K, _ = fx.make_attn(w)
    p = problem(w)
    st = tka().topk_attn_score(p, dev(q), dev(K))
    s = gpu_scores_np(st).reshape(-1, w.L).astype(np.float32)
    idx, k, tau, sel = run_select(st.reshape(s.shape[0], -1), float(eps), 1, kmax)
    check_rows(s, float(eps), 1, kmax, idx, k, tau)
    rows = np.arange(s.shape[0])
    for r in rows:
        kk = int(k[r])
        assert np.array_equal(sel[r, :kk].view(np.uint32), s[r, idx[r, :kk]].view(np.uint32))
        assert np.all(np.isneginf(sel[r, kk:]))
    say(f"[adaptive] {name} L={L} eps={float(eps)}: k mean {k.mean():.1f} min {k.min()} max {k.max()}")


def edge_rows(n):
    rng = np.random.default_rng(5)
    rows = []
    rows.append(np.full(n, 0.25, np.float32))                      # uniform: ceil((1 - eps) n)
    one = np.full(n, -np.inf, np.float32)
    one[n // 3] = 2.0
    rows.append(one)                                               # all mass on one key
    rows.append(np.full(n, np.nan, np.float32))                    # no mass
    rows.append(np.full(n, -np.inf, np.float32))                   # maximum -inf: every key has mass 1
    x = rng.normal(size=n).astype(np.float32)
    x[::7] = np.inf                                                # +inf keys share the mass
    rows.append(x)
    rows.append(np.round(rng.normal(size=n) * 2).astype(np.float32))  # heavy ties
    st = np.repeat(np.arange(n // 8, dtype=np.float32), 8)[:n][::-1].copy()  # staircase of runs
    rows.append(np.resize(st, n))
    y = rng.normal(size=n).astype(np.float32) * 30                 # very peaked, many tiny masses
    y[rng.integers(0, n, 10)] = np.nan
    rows.append(y)
    z = rng.normal(size=n).astype(np.float32)
    z[z > 0] = -0.0
    rows.append(z)                                                 # -0 / +0 ties at the top
    return np.stack(rows)


@pytest.mark.parametrize("n", [1, 37, 1000, 4099, 20000, 65536])  # the last two: the sampled path of long rows
@pytest.mark.parametrize("eps,k_min,k_max", [(0.0, 1, 5000), (0.05, 1, 5000), (0.3, 4, 9), (0.999, 2, 5000),
                                             (0.2, 0, 3)])
def test_adaptive_select_edge_rows(n, eps, k_min, k_max):
    s = edge_rows(n)
    idx, k, tau, _ = run_select(dev(s), eps, k_min, k_max)
    check_rows(s, eps, k_min, k_max, idx, k, tau)
    # rows with an exact answer
    lo, hi = max(k_min, 1), min(k_max, n)
    clamp = lambda v: min(max(v, lo), hi)
    e32 = float(np.float32(eps))
    assert k[0] == clamp(math.ceil((1 - e32) * n - 1e-9))  # uniform: ceil((1 - eps) n)
    assert k[1] == clamp(1) and n // 3 in idx[1, :k[1]]    # all the mass on one key
    assert k[2] == min(lo, hi) and math.isnan(tau[2])      # no mass


def test_adaptive_select_empty_rows_and_checks():
    m = tka()
    s = torch.empty((3, 0), dtype=torch.float32, device="cuda")
    idx, k, tau, _ = m.topk_select_adaptive(s, 0.1, 1, 4, row_len=0, row_stride=0)
    torch.cuda.synchronize()
    assert torch.all(idx == -1) and torch.all(k == 0) and torch.all(torch.isnan(tau))
    with pytest.raises(m.TkaError):
        m.topk_select_adaptive(torch.zeros((2, 8), device="cuda"), float("nan"), 1, 4)
    with pytest.raises(m.TkaError):
        m.topk_select_adaptive(torch.zeros((2, 8), device="cuda"), -0.5, 1, 4)


CASES = {
    "C2-small": fx.shrink(fx.WORKLOADS["C2"], 6001, k=1024),
    "f32-d64": fx.Workload("exact-f32-d64-g2", fx.MODE_EXACT, 2, 4, 2, 64, 3000, 512, fx.F32, 41,
                           fx.PLANT_SCALE, 30, 3.0),
    "C3-small": fx.shrink(fx.WORKLOADS["C3"], 12000, B=1, k=2048),
}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("eps", [0.02, 0.2])
def test_adaptive_decode_against_oracle_and_composition(name, eps):
    w = CASES[name]
    m = tka()
    q, K, V = fx.make_attn(w)
    qt, Kt, Vt = dev(q), dev(K), dev(V)
    p = problem(w)
    out, idx, k, tau = m.topk_decode_adaptive(p, qt, Kt, Vt, eps, 1)
    out2, idx2, k2, tau2 = m.topk_decode_adaptive(p, qt, Kt, Vt, eps, 1)
    st = m.topk_attn_score(p, qt, Kt)
    rows = w.B * w.Hq
    ci, ck, ct, cs = m.topk_select_adaptive(st.reshape(rows, -1), eps, 1, w.k, want_sel=True)
    co = m.sparse_attn_gather(p, qt, Kt, Vt, ci.reshape(w.B, w.Hq, w.k), sel_scores=cs.reshape(w.B, w.Hq, w.k))
    torch.cuda.synchronize()
    assert torch.equal(idx.reshape(rows, -1), ci) and torch.equal(k.reshape(-1), ck)
    assert torch.equal(tau.reshape(-1).view(torch.int32), ct.view(torch.int32))
    assert torch.equal(out.view(torch.int32), co.view(torch.int32))
    assert torch.equal(out2.view(torch.int32), out.view(torch.int32)) and torch.equal(idx2, idx)
    s = gpu_scores_np(st).reshape(rows, -1).astype(np.float32)
    gi, gk, gt = idx.cpu().numpy().reshape(rows, -1), k.cpu().numpy().reshape(-1), tau.cpu().numpy().reshape(-1)
    check_rows(s, eps, 1, w.k, gi, gk, gt)
    ref = orc.attend(orc.problem_for(w), q, K, V, gi, list_mode=0)
    got = out.cpu().numpy().reshape(rows, -1).astype(np.float64)
    assert np.abs(got - ref).max() <= tol(w), float(np.abs(got - ref).max())
    say(f"[adaptive decode] {name} eps={eps}: k mean {gk.mean():.1f}, tau max {gt.max():.4f}")
