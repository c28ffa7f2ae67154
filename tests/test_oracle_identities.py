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
