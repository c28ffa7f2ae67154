"""Pins of the oracle's top-k selection.

TopK over scores ("Sparse Attention Landscape", "Block Sparse Attention",
TopK_j s_j) keeps the k highest. Readings fixed for a unique answer: ties go to
the lower position, NaN ranks below every number, -0 == +0, output ascending,
-1 padding when k > row length (the fixed budget means at most k positions,
"Sparse Attention in LLM Inference", "The Significance of Top-K").

Pins: brute-force dominance on tiny rows (every kept element outranks every
dropped one), numpy's lexsort as an independent library order, and special
cases with a known answer.
"""
import itertools
import math

import numpy as np
import pytest

import oracle as orc


def _outranks(a, ia, b, ib):
    """a at position ia ranks above b at position ib."""
    an, bn = math.isnan(a), math.isnan(b)
    if an != bn:
        return bn
    if not an and a != b:
        return a > b
    return ia < ib


def _check_row(row, k, got):
    L = len(row)
    kk = min(k, L)
    kept = list(got[:kk])
    assert all(x == -1 for x in got[kk:])
    assert kept == sorted(kept) and len(set(kept)) == kk
    assert all(0 <= x < L for x in kept)
    ks = set(kept)
    for i in ks:
        for j in range(L):
            if j not in ks:
                assert _outranks(row[i], i, row[j], j), (row, k, got)


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_bruteforce_dominance_tiny_rows(dtype):
    rng = np.random.default_rng(7)
    pool = np.array([-2.0, -1.0, -0.0, 0.0, 1.0, 2.0, np.inf, -np.inf, np.nan, 0.5])
    for L in range(1, 13):
        rows = rng.choice(pool, size=(6, L)).astype(dtype)
        for k in range(1, L + 3):
            idx = orc.select(rows, k)
            for r in range(rows.shape[0]):
                _check_row([float(x) for x in rows[r]], k, idx[r])


def test_subset_enumeration_tiny():
    """For L <= 8 the kept set is the only k-subset that outranks its complement."""
    rng = np.random.default_rng(3)
    for L in range(1, 9):
        row = rng.integers(0, 3, L).astype(np.float64)
        for k in range(1, L + 1):
            got = set(orc.select(row, k)[0].tolist())
            ok = [set(c) for c in itertools.combinations(range(L), k)
                  if all(_outranks(row[i], i, row[j], j) for i in c for j in range(L) if j not in c)]
            assert ok == [got]


def test_against_numpy_lexsort():
    rng = np.random.default_rng(11)
    for L, k in [(1000, 64), (4097, 300), (2047, 16)]:
        s = np.round(rng.standard_normal((4, L)), 2)  # many duplicates
        idx = orc.select(s, k)
        for r in range(4):
            order = np.lexsort((np.arange(L), -s[r]))  # primary -s, secondary position
            assert np.array_equal(idx[r], np.sort(order[:k]))


def test_f32_and_f64_paths_agree():
    rng = np.random.default_rng(5)
    s = rng.standard_normal((3, 5000)).astype(np.float32)
    assert np.array_equal(orc.select(s, 123), orc.select(s.astype(np.float64), 123))


def test_special_cases():
    L = 100
    # all equal -> the k lowest positions
    assert orc.select(np.full(L, 0.25), 10)[0].tolist() == list(range(10))
    # k = L keeps all, k > L pads with -1
    row = np.random.default_rng(0).standard_normal(L)
    assert orc.select(row, L)[0].tolist() == list(range(L))
    assert orc.select(row, L + 5)[0].tolist() == list(range(L)) + [-1] * 5
    # k = 1 -> lowest-index argmax
    r2 = np.array([1.0, 3.0, 2.0, 3.0, -5.0])
    assert orc.select(r2, 1)[0].tolist() == [1]
    # +0 and -0 tie; the lower index wins
    assert orc.select(np.array([-0.0, 0.0, -1.0]), 1)[0].tolist() == [0]
    assert orc.select(np.array([0.0, -0.0, -1.0]), 1)[0].tolist() == [0]
    # NaN below -inf
    assert orc.select(np.array([np.nan, -np.inf, np.nan]), 2)[0].tolist() == [0, 1]
    # staircase with a run of equal values across the threshold
    st = np.array([5, 5, 4, 4, 4, 4, 3, 3], np.float64)
    assert orc.select(st, 4)[0].tolist() == [0, 1, 2, 3]


def test_values_sharing_high_key_bits():
    """Values equal in their top 20 bits still order exactly (fp32 bit patterns)."""
    base = np.float32(1.5).view(np.uint32)
    bits = base + np.arange(0, 4096, dtype=np.uint32)[::-1]  # distinct low bits
    row = bits.view(np.float32)
    rng = np.random.default_rng(1)
    perm = rng.permutation(len(row))
    sh = row[perm]
    idx = orc.select(sh, 37)[0]
    want = np.sort(np.argsort(-sh.astype(np.float64), kind="stable")[:37])
    assert np.array_equal(idx, want)
