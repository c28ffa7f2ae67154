"""Pins from "A Mathematical Theory of Top-k Sparse Attention via Total
Variation Distance" (abstract):

- TV(P, P-hat) equals the discarded softmax tail mass tau and equals
  1 - exp(-KL(P-hat || P)).
- Head-tail factorisation: ||Attn - Attn_k||_2 = tau * ||mu_tail - mu_head||_2,
  and the head-tail diameter bound ||Attn - Attn_k||_2 <= tau * diam(H, T)
  (read as the cross diameter over kept x dropped value rows).
- Gaussian score model s_i ~ N(mu, sigma^2): the tail mass kept by the top
  fraction f is closed-form, tau = Phi(Phi^-1(1 - f) - sigma), and the
  minimal k for TV <= eps satisfies k_eps / n ~ Phi^c(sigma + Phi^-1(eps)).

Dense attention (Attn) comes from torch's SDPA (library), the top-k output
(Attn_k) from the oracle's decode path, the distribution quantities from the
oracle's diagnostics.
"""
import numpy as np
import pytest
import torch
from scipy.stats import norm

import fixtures as fx
import oracle as orc


def _dense(q, K, V, b, h, G):
    qt = torch.from_numpy(q[b, h].astype(np.float64))[None, None, None, :]
    Kt = torch.from_numpy(K[b, h // G].astype(np.float64))[None, None]
    Vt = torch.from_numpy(V[b, h // G].astype(np.float64))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt)[0, 0, 0].numpy()


@pytest.mark.parametrize("name,L", [("C1", 1024), ("C2", 1500), ("C4", 2000)])
def test_tv_tail_kl_and_head_tail(name, L):
    w = fx.shrink(fx.WORKLOADS[name], L, B=1, Hq=4, Hkv=2) if name != "C1" else fx.WORKLOADS[name]
    # use the exact variant of every recipe
    p = orc.problem(orc.EXACT, w.B, w.Hq, w.Hkv, w.d, w.L, min(w.k, w.L // 4), w.dtype)
    q, K, V = fx.make_attn(w)
    out, idx = orc.decode(p, q, K, V)
    qf = q.astype(np.float32) if w.dtype == fx.F32 else fx.bf16_bits_to_f32(q)
    Kf = K.astype(np.float32) if w.dtype == fx.F32 else fx.bf16_bits_to_f32(K)
    Vf = V.astype(np.float32) if w.dtype == fx.F32 else fx.bf16_bits_to_f32(V)
    for r in range(min(p.B * p.Hq, 4)):
        b, h = divmod(r, p.Hq)
        dg = orc.diag_exact(p, q, K, V, r, idx[r])
        tau, tv, kl = dg["tau"], dg["tv"], dg["kl"]
        assert abs(tv - tau) < 1e-12
        assert abs(tv - (1 - np.exp(-kl))) < 1e-12
        full = _dense(qf, Kf, Vf, b, h, p.Hq // p.Hkv)
        assert np.abs(full - dg["o_full"]).max() < 1e-12
        # the top-k output is the head mean
        assert np.abs(out[r] - dg["mu_head"]).max() < 1e-12
        err = np.linalg.norm(full - out[r])
        assert abs(err - tau * np.linalg.norm(dg["mu_tail"] - dg["mu_head"])) < 1e-12
        if np.isfinite(dg["diam"]):
            assert err <= tau * dg["diam"] + 1e-12


def test_tail_mass_falls_as_k_grows():
    w = fx.shrink(fx.WORKLOADS["C2"], 2000, B=1, Hq=4, Hkv=1)
    q, K, V = fx.make_attn(w)
    taus = []
    for k in [1, 10, 100, 1000, 2000]:
        p = orc.problem(orc.EXACT, 1, 4, 1, 128, 2000, k, fx.BF16)
        _, idx = orc.decode(p, q, K, V, rows=[0])
        taus.append(orc.diag_exact(p, q, K, V, 0, idx[0])["tau"])
    assert all(a >= b for a, b in zip(taus, taus[1:]))
    assert taus[-1] == 0.0


def test_gaussian_tail_mass_and_k_eps():
    """Unplanted fp32 keys: s_i | q is exactly N(0, ||q||^2 / d)."""
    d, L = 64, 131072
    q = fx.normal(101, 0, d).reshape(1, 1, d)
    K = fx.normal(101, 1, L * d).reshape(1, 1, L, d)
    V = fx.normal(101, 2, L * d).reshape(1, 1, L, d)
    sigma = float(np.linalg.norm(q.astype(np.float64)) / np.sqrt(d))
    for f in [1 / 32, 1 / 16, 1 / 8]:
        k = int(L * f)
        p = orc.problem(orc.EXACT, 1, 1, 1, d, L, k, orc.F32)
        _, idx = orc.decode(p, q, K, V)
        tau = orc.diag_exact(p, q, K, V, 0, idx[0])["tau"]
        assert abs(tau - norm.cdf(norm.ppf(1 - f) - sigma)) < 0.01
    # k_eps from the oracle's sorted probability mass
    p = orc.problem(orc.EXACT, 1, 1, 1, d, L, L, orc.F32)
    s = orc.score(p, q, K)[0]
    P = np.exp(s - s.max())
    P = np.sort(P / P.sum())[::-1]
    kept = np.cumsum(P)
    for eps in [0.1, 0.05, 0.01]:
        k_eps = int(np.argmax(1 - kept <= eps)) + 1
        pred = norm.sf(sigma + norm.ppf(eps)) * L
        assert abs(k_eps - pred) / pred < 0.02


# ---- entropy H(P) and boundary gap s_(k') - s_(k'+1) of the diagnostics ----
# "A Preliminary Study on the Promises and Challenges of Native Top-k Sparse
# Attention" (abstract) ties top-k suitability to low attention entropy; the
# boundary gap is the margin between the last kept and the first dropped score.
# Pins: rows whose scores take one or two values (H in closed form via
# H = ln Z - E_P[s], gap = a - b exactly), a one-hot row (H -> 0), and random
# rows checked against scipy's entropy of scipy's softmax and a numpy sort.

def _two_value_row(L, n_hi, a, b, d=16, seed=7):
    """fp32 row with q = e_0 and scale 1: s_i = K[i, 0] exactly, a on n_hi positions, b elsewhere."""
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 0] = 1.0
    K = fx.normal(seed, 1, L * d).reshape(1, 1, L, d)
    hi = fx.sample_distinct(seed, 3, L, n_hi) if n_hi else np.zeros(0, np.int64)
    K[0, 0, :, 0] = b
    K[0, 0, hi, 0] = a
    V = fx.normal(seed, 2, L * d).reshape(1, 1, L, d)
    return q, K, V, np.sort(hi)


def _h_closed(n_hi, a, n_lo, b):
    # H = ln Z - E_P[s] with Z = sum e^{s_i}, shifted by the maximum for range
    m = max(a if n_hi else -np.inf, b if n_lo else -np.inf)
    ea, eb = n_hi * np.exp(a - m), n_lo * np.exp(b - m)
    Z = ea + eb
    return np.log(Z) + m - (a * ea + b * eb) / Z


@pytest.mark.parametrize("L,n_hi,a,b", [(1000, 37, 2.5, -0.75), (4096, 1, 3.0, 0.0), (777, 400, -1.25, -3.5)])
def test_entropy_and_gap_two_value_rows(L, n_hi, a, b):
    q, K, V, hi = _two_value_row(L, n_hi, a, b)
    p = orc.problem(orc.EXACT, 1, 1, 1, 16, L, n_hi, orc.F32, scale=1.0)
    dg = orc.diag_exact(p, q, K, V, 0, hi.astype(np.int32))
    assert abs(dg["entropy"] - _h_closed(n_hi, a, L - n_hi, b)) < 1e-12
    assert dg["gap"] == a - b          # kept set = exactly the high positions
    # a kept set inside the high tier, or reaching into the low tier: the boundary scores are equal
    if n_hi > 1:
        assert orc.diag_exact(p, q, K, V, 0, hi[:-1].astype(np.int32))["gap"] == 0.0
    lo = np.setdiff1d(np.arange(L), hi)[:3]
    assert orc.diag_exact(p, q, K, V, 0, np.concatenate([hi, lo]).astype(np.int32))["gap"] == 0.0
    # everything kept: no dropped score, the gap is +inf and nothing is discarded
    everything = orc.diag_exact(p, q, K, V, 0, np.arange(L, dtype=np.int32))
    assert everything["gap"] == np.inf and everything["tau"] == 0.0


def test_entropy_uniform_row_is_log_L():
    """Every key equal: P is uniform, H = ln L, every boundary gap 0."""
    d, L = 32, 3001
    q = fx.normal(9, 0, d).reshape(1, 1, d)
    row = fx.normal(9, 1, d)
    K = np.broadcast_to(row, (1, 1, L, d)).copy()
    V = fx.normal(9, 2, L * d).reshape(1, 1, L, d)
    p = orc.problem(orc.EXACT, 1, 1, 1, d, L, 100, orc.F32)
    dg = orc.diag_exact(p, q, K, V, 0, np.arange(100, dtype=np.int32))
    assert abs(dg["entropy"] - np.log(L)) < 1e-12
    assert dg["gap"] == 0.0
    assert abs(dg["tau"] - (L - 100) / L) < 1e-12


def test_entropy_one_hot_row_vanishes():
    """One score 60 above all others: P is one-hot up to e^-60, so H is about L e^-60 * 61."""
    L = 2048
    q, K, V, hi = _two_value_row(L, 1, 60.0, 0.0)
    p = orc.problem(orc.EXACT, 1, 1, 1, 16, L, 1, orc.F32, scale=1.0)
    dg = orc.diag_exact(p, q, K, V, 0, hi.astype(np.int32))
    assert 0.0 <= dg["entropy"] < 1e-20
    assert dg["gap"] == 60.0
    assert dg["tau"] < 1e-22


@pytest.mark.parametrize("name,k", [("C1", 64), ("C2", 300)])
def test_entropy_and_gap_on_workload_rows(name, k):
    """Random workload rows: H equals scipy's entropy of scipy's softmax of numpy's fp64 scores, and the gap
    equals the difference of the k-th and (k+1)-th largest of those scores."""
    from scipy.special import softmax
    from scipy.stats import entropy
    w = fx.WORKLOADS[name] if name == "C1" else fx.shrink(fx.WORKLOADS[name], 3000, B=1, Hq=4, Hkv=1)
    q, K, V = fx.make_attn(w)
    p = orc.problem(orc.EXACT, w.B, w.Hq, w.Hkv, w.d, w.L, k, w.dtype)
    _, idx = orc.decode(p, q, K, V)
    qf = q.astype(np.float64) if w.dtype == fx.F32 else fx.bf16_bits_to_f32(q).astype(np.float64)
    Kf = K.astype(np.float64) if w.dtype == fx.F32 else fx.bf16_bits_to_f32(K).astype(np.float64)
    for r in range(w.B * w.Hq):
        b, h = divmod(r, w.Hq)
        s = (Kf[b, h // w.G] @ qf[b, h]) / np.sqrt(w.d)
        dg = orc.diag_exact(p, q, K, V, r, idx[r])
        assert abs(dg["entropy"] - entropy(softmax(s))) < 1e-9
        srt = np.sort(s)[::-1]
        assert abs(dg["gap"] - (srt[k - 1] - srt[k])) < 1e-12


# ---- the Gaussian rule at the workloads' own shapes (bf16 keys, d = 128) ----
# Unplanted twins of the exact-variant workloads: N(0,1) bf16 q, K, V, the
# configs' k and L. For bf16 keys s_i given q is very nearly N(0, ||q||^2/d), so
# the realised discarded mass follows tau = Phi(Phi^-1(1 - k/L) - sigma) and the
# smallest k meeting TV <= eps follows k_eps/L = Phi^c(sigma + Phi^-1(eps))
# ("A Mathematical Theory of Top-k Sparse Attention via Total Variation
# Distance", abstract).

@pytest.mark.parametrize("name,L,k,heads", [("C2", 32768, 2048, 4), ("C3", 131072, 4096, 4),
                                            ("C5", 1048576, 2048, 2)])
def test_gaussian_rule_bf16_workload_shapes(name, L, k, heads):
    w = fx.Workload(name + "-unplanted", fx.MODE_EXACT, 1, heads, 1, 128, L, k, fx.BF16,
                    1000 + int(name[1]))
    q, K, V = fx.make_attn(w)
    p = orc.problem(orc.EXACT, 1, heads, 1, 128, L, k, fx.BF16)
    s = orc.score(p, q, K)
    idx = orc.select(s, k)
    for h in range(heads):
        sigma = float(np.linalg.norm(fx.bf16_bits_to_f32(q[0, h]).astype(np.float64)) / np.sqrt(128))
        tau = orc.diag_exact(p, q, K, V, h, idx[h])["tau"]
        assert abs(tau - norm.cdf(norm.ppf(1 - k / L) - sigma)) < 0.01
        P = np.exp(s[h] - s[h].max())
        kept = np.cumsum(np.sort(P / P.sum())[::-1])
        for eps in [0.1, 0.05, 0.01]:
            k_eps = int(np.argmax(1 - kept <= eps)) + 1
            pred = norm.sf(sigma + norm.ppf(eps)) * L
            assert abs(k_eps - pred) / pred < 0.02
