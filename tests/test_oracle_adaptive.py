"""Pins of the oracle's certified adaptive top-k (the smallest k whose top-k
keeps at least 1 - eps of the softmax mass; "A Mathematical Theory of Top-k
Sparse Attention via Total Variation Distance", abstract: TV(P, P-hat) is the
discarded tail mass, and k_eps/n ~ Phi^c(sigma + Phi^-1(eps)) for i.i.d.
Gaussian logits).

Checked against: enumeration of every k on tiny rows, the closed form for
uniform logits, the page's Gaussian rule at large n, the oracle's separate
diagnostics routine (tau and TV of the returned set), and degenerate rows."""
import math

import numpy as np
import pytest
from scipy.stats import norm

import fixtures as fx
import oracle as orc


def brute(row, eps, k_min, k_max):
    """Every k from 1 up: the discarded mass of the first k in the select order."""
    n = len(row)
    v = row.astype(np.float64)
    order = sorted(range(n), key=lambda i: (math.isnan(v[i]), -v[i] if not math.isnan(v[i]) else 0.0, i))
    finite = v[~np.isnan(v)]
    M = finite.max()
    w = np.array([0.0 if math.isnan(x) else (1.0 if x == M else math.exp(x - M)) for x in v])
    Z = w.sum()
    k = n
    for kk in range(0, n + 1):
        if w[order[kk:]].sum() <= eps * Z:
            k = kk
            break
    k = min(max(k, max(k_min, 1)), min(k_max, n))
    return sorted(order[:k]), k, w[order[k:]].sum() / Z


@pytest.mark.parametrize("seed", range(8))
def test_tiny_rows_against_enumeration(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 24))
    row = rng.normal(size=n) * rng.uniform(0.2, 4.0)
    if seed % 2:  # many ties
        row = np.round(row)
    row = row.astype(np.float32)
    for eps in (0.0, 0.01, 0.1, 0.5, 0.99):
        for k_min, k_max in ((1, n), (2, n + 3), (1, max(1, n // 2))):
            idx, k, tau = orc.select_adaptive(row, eps, k_min, k_max)
            want_idx, want_k, want_tau = brute(row, eps, k_min, k_max)
            assert k[0] == want_k, (eps, k_min, k_max)
            assert list(idx[0, :k[0]]) == want_idx and np.all(idx[0, k[0]:] == -1)
            assert abs(tau[0] - want_tau) <= 1e-15


def test_uniform_logits_closed_form():
    # P_i = 1/n: the top k keeps k/n, so k_eps = ceil((1 - eps) n)
    for n, eps in ((1000, 0.0123), (4097, 0.3), (50, 0.071)):
        row = np.full(n, 0.75, np.float32)
        idx, k, tau = orc.select_adaptive(row, eps, 1, n)
        want = math.ceil((1 - eps) * n)
        assert k[0] == want
        assert list(idx[0, :want]) == list(range(want))  # ties go to the lower positions
        assert abs(tau[0] - (n - want) / n) <= 1e-12


@pytest.mark.parametrize("sigma,eps", [(1.0, 0.05), (1.0, 0.1), (1.5, 0.05), (0.5, 0.01)])
def test_gaussian_rule_for_k_eps(sigma, eps):
    n = 1 << 18
    row = (fx.normal(31, 0, n) * sigma).astype(np.float64)
    _, k, tau = orc.select_adaptive(row, eps, 1, n)
    predicted = norm.sf(sigma + norm.ppf(eps))
    assert abs(k[0] / n - predicted) <= 0.02 * predicted, (k[0] / n, predicted)
    assert tau[0] <= eps


def test_tau_matches_diagnostics_of_the_returned_set():
    w = fx.shrink(fx.WORKLOADS["C1"], 1024)
    q, K, V = fx.make_attn(w)
    p = orc.problem_for(w)
    s = orc.score(p, q, K)
    for eps in (0.02, 0.2):
        idx, k, tau = orc.select_adaptive(s, eps, 1, w.L)
        kept = idx[0, :k[0]]
        d = orc.diag_exact(p, q, K, V, 0, kept)
        assert abs(d["tau"] - tau[0]) <= 1e-12 and abs(d["tv"] - tau[0]) <= 1e-12
        assert tau[0] <= eps
        if k[0] > 1:  # one fewer key would break the budget
            _, _, tau_less = orc.select_adaptive(s, eps, 1, int(k[0]) - 1)
            assert tau_less[0] > eps


def test_degenerate_and_clamped_rows():
    n = 64
    one = np.full(n, -np.inf, np.float32)
    one[17] = 3.0  # all the mass on one key
    idx, k, tau = orc.select_adaptive(one, 0.0, 1, 8)
    assert k[0] == 1 and idx[0, 0] == 17 and tau[0] == 0.0 and np.all(idx[0, 1:] == -1)
    # k_min forces more keys than the budget needs; k_max caps below it
    row = fx.normal(32, 0, n).astype(np.float32)
    _, k_free, _ = orc.select_adaptive(row, 0.3, 1, n)
    _, k_lo, tau_lo = orc.select_adaptive(row, 0.3, int(k_free[0]) + 5, n)
    assert k_lo[0] == k_free[0] + 5 and tau_lo[0] < 0.3
    _, k_hi, tau_hi = orc.select_adaptive(row, 0.3, 1, int(k_free[0]) - 3)
    assert k_hi[0] == k_free[0] - 3 and tau_hi[0] > 0.3
    # NaN scores carry no mass and rank last; a row of NaN keeps k_min keys with tau NaN
    nan = np.full(n, np.nan, np.float32)
    idx, k, tau = orc.select_adaptive(nan, 0.1, 3, 8)
    assert k[0] == 3 and list(idx[0, :3]) == [0, 1, 2] and math.isnan(tau[0])
    # eps >= 1 needs no mass at all: the clamp floor
    _, k, tau = orc.select_adaptive(row, 1.0, 1, n)
    assert k[0] == 1
