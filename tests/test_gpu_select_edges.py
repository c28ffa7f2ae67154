"""GPU top-k select on adversarial rows, bit-exact against the oracle's select
on the same fp32 array: ties across the threshold (lower index wins), +-0,
+-inf, NaN (below -inf), all-equal rows, values sharing their top 20 bits
(forces every radix level), sorted rows (candidates all in one wave), huge
tie runs (streaming emit), k = 1, k = n - 1, k = n, k > n, empty rows, rows
with a stride, and every launch shape (one workgroup per row, 256 or 1024 threads; chunked rows)."""
import zlib

import numpy as np
import pytest
import torch

import oracle as orc
from tests.gpu_common import say, tka

pytestmark = pytest.mark.gpu


def _rows(kind, n_rows, n, rng):
    if kind == "normal":
        return rng.standard_normal((n_rows, n)).astype(np.float32)
    if kind == "dups":
        return np.round(rng.standard_normal((n_rows, n)), 1).astype(np.float32)
    if kind == "equal":
        return np.full((n_rows, n), 0.75, np.float32)
    if kind == "zeros":
        return rng.choice(np.array([0.0, -0.0, -1.0, 1.0], np.float32), size=(n_rows, n))
    if kind == "special":
        x = rng.standard_normal((n_rows, n)).astype(np.float32)
        m = rng.random((n_rows, n))
        x[m < 0.02] = np.inf
        x[(m >= 0.02) & (m < 0.05)] = -np.inf
        x[(m >= 0.05) & (m < 0.09)] = np.nan
        x[(m >= 0.09) & (m < 0.12)] = -0.0
        return x
    if kind == "lowbits":
        bits = np.uint32(0x3FC00000) + rng.integers(0, 1 << 12, size=(n_rows, n)).astype(np.uint32)
        return bits.view(np.float32)
    if kind == "ascending":
        return np.tile(np.arange(n, dtype=np.float32), (n_rows, 1))
    if kind == "descending":
        return np.tile(-np.arange(n, dtype=np.float32), (n_rows, 1))
    if kind == "tierun":  # a long run of one value straddles the threshold
        x = rng.standard_normal((n_rows, n)).astype(np.float32)
        x[:, rng.random(n) < 0.6] = 0.5
        return x
    if kind == "staircase":
        return np.tile(np.repeat(np.arange(n // 7 + 1, dtype=np.float32)[::-1], 7)[:n], (n_rows, 1))
    if kind == "skew":  # the large values crowd into the first eighth of the row
        x = rng.standard_normal((n_rows, n)).astype(np.float32)
        x[:, : n // 8] += 3.0
        return x
    raise ValueError(kind)


def _seed(kind, n):  # stable across processes (str hashes are salted per process)
    return zlib.crc32(f"{kind}/{n}".encode())


KINDS = ["normal", "dups", "equal", "zeros", "special", "lowbits", "ascending", "descending", "tierun", "staircase"]
# row mode x2, one 1024-thread workgroup per row (a few rows of 8193..32768) x3, chunked mode x2
SHAPES = [(200, 3000), (130, 20000), (7, 9001), (100, 20000), (5, 32768), (3, 70001), (1, 300000)]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("shape", SHAPES)
def test_select_adversarial(kind, shape):
    n_rows, n = shape
    rng = np.random.default_rng(_seed(kind, n))
    x = _rows(kind, n_rows, n, rng)
    xt = torch.from_numpy(x).cuda()
    m = tka()
    for k in sorted({1, 37, n // 33 + 1, 2048, n - 1, n, n + 5}):
        say(f"[select edges] {kind} {shape} k={k}")
        idx, sel = m.topk_select(xt, k)
        idx2, sel2 = m.topk_select(xt, k)
        gi = idx.cpu().numpy()
        want = orc.select(x, k)
        assert np.array_equal(gi, want), (kind, shape, k)
        kk = min(k, n)
        rows = np.arange(n_rows)[:, None]
        gs = sel.cpu().numpy()
        assert np.array_equal(gs[:, :kk].view(np.uint32), x[rows, gi[:, :kk]].view(np.uint32))
        assert np.all(np.isneginf(gs[:, kk:]))
        assert torch.equal(idx, idx2) and torch.equal(sel.view(torch.int32), sel2.view(torch.int32))


@pytest.mark.parametrize("kind", ["normal", "dups", "tierun", "ascending", "special", "skew", "equal"])
def test_select_long_rows_sampled_threshold(kind):
    """Rows of 131072 with k' <= n/8 take the sampled threshold and one collecting pass; rows
    where it cannot hold (ties, crowding) fall back to the digit search: bit-exact either way."""
    n_rows, n = 128, 131072
    rng = np.random.default_rng(_seed(kind, "long"))
    x = _rows(kind, n_rows, n, rng)
    xt = torch.from_numpy(x).cuda()
    m = tka()
    for k in (512, 4096):
        say(f"[select long rows] {kind} k={k}")
        idx, sel = m.topk_select(xt, k)
        gi = idx.cpu().numpy()
        assert np.array_equal(gi, orc.select(x, k)), (kind, k)
        rows = np.arange(n_rows)[:, None]
        assert np.array_equal(sel.cpu().numpy().view(np.uint32), x[rows, gi].view(np.uint32))


def test_select_strided_and_unaligned_rows():
    rng = np.random.default_rng(5)
    base = torch.from_numpy(rng.standard_normal((64, 5003)).astype(np.float32)).cuda()
    view = base[:, 1:4001]  # rows start 4 bytes off 16-byte alignment, stride 5003
    m = tka()
    idx, _ = m.topk_select(view, 100, row_len=4000, row_stride=5003)
    want = orc.select(base.cpu().numpy()[:, 1:4001].copy(), 100)
    assert np.array_equal(idx.cpu().numpy(), want)
    # a few long rows (one 1024-thread workgroup per row), off alignment, with NaN and -0 kept
    x = rng.standard_normal((8, 20003)).astype(np.float32)
    x[:, ::97] = np.nan
    x[:, 5::89] = -0.0
    x[:, 7::101] = 0.0
    wide = torch.from_numpy(x).cuda()
    for k in (3000, 20000):
        idx, sel = m.topk_select(wide[:, 1:20002], k, row_len=20001, row_stride=20003)
        xs = x[:, 1:20002].copy()
        gi = idx.cpu().numpy()
        assert np.array_equal(gi, orc.select(xs, k)), k
        assert np.array_equal(sel.cpu().numpy().view(np.uint32), xs[np.arange(8)[:, None], gi].view(np.uint32))


def test_select_empty_rows_pad():
    m = tka()
    x = torch.empty((4, 0), dtype=torch.float32, device="cuda")
    idx, sel = m.topk_select(x, 8, row_len=0, row_stride=0)
    assert (idx.cpu() == -1).all() and torch.isneginf(sel.cpu()).all()


# short rows with k <= 64 take the one-wave-per-row kernel (n <= 2048); n = 2049 and k = 65 the others
SHORT_SHAPES = [(128, 2047), (5, 2048), (3, 2049), (70, 64), (3, 63), (2, 1), (9, 1000), (6, 130)]


@pytest.mark.parametrize("kind", KINDS + ["skew"])
@pytest.mark.parametrize("shape", SHORT_SHAPES)
def test_select_short_rows(kind, shape):
    n_rows, n = shape
    rng = np.random.default_rng(_seed(kind, n) + 1)
    x = _rows(kind, n_rows, n, rng)
    xt = torch.from_numpy(x).cuda()
    m = tka()
    for k in sorted({1, 2, 16, 37, 63, 64, 65, n - 1, n, n + 5} - {0}):
        if k > 65:
            continue
        say(f"[select short] {kind} {shape} k={k}")
        idx, sel = m.topk_select(xt, k)
        gi = idx.cpu().numpy()
        assert np.array_equal(gi, orc.select(x, k)), (kind, shape, k)
        kk = min(k, n)
        rows = np.arange(n_rows)[:, None]
        gs = sel.cpu().numpy()
        assert np.array_equal(gs[:, :kk].view(np.uint32), x[rows, gi[:, :kk]].view(np.uint32))
        assert np.all(np.isneginf(gs[:, kk:]))


def test_select_short_rows_strided():
    """Rows of a wider array (row stride > row length), as the block-mean scores are read."""
    rng = np.random.default_rng(7)
    full = np.round(rng.standard_normal((64, 2100)), 1).astype(np.float32)
    n = 2047
    xt = torch.from_numpy(full).cuda()
    m = tka()
    for k in (1, 16, 64):
        say(f"[select short strided] k={k}")
        idx, _ = m.topk_select(xt, k, row_len=n, row_stride=2100)
        assert np.array_equal(idx.cpu().numpy(), orc.select(full[:, :n], k))


def test_select_many_long_rows_hot_samples_and_strides():
    """Many long rows take the candidate select (samples -> per-row threshold -> one collecting
    pass over all rows -> select among the candidates). Scores planted high exactly on the sampled
    runs (32 runs of 64 starting at j n / 32) put the threshold above the k'-th score, so those rows
    have too few candidates and take the full row select; a padded stride, rows starting off 16-byte
    alignment (the row kernel instead) and exactly 64 rows are covered too. Bit-exact throughout."""
    m = tka()
    rng = np.random.default_rng(41)
    n_rows, n, k = 96, 32768, 2048
    x = rng.standard_normal((n_rows, n)).astype(np.float32)
    for r in range(0, n_rows, 3):  # every third row: the sampled runs hold the largest values
        for j in range(32):
            at = j * n // 32
            x[r, at:at + 64] = 50.0 + rng.random(64).astype(np.float32)
    say("[select many rows] hot samples")
    idx, sel = m.topk_select(torch.from_numpy(x).cuda(), k)
    gi = idx.cpu().numpy()
    assert np.array_equal(gi, orc.select(x, k))
    rows = np.arange(n_rows)[:, None]
    assert np.array_equal(sel.cpu().numpy().view(np.uint32), x[rows, gi].view(np.uint32))

    flat = torch.from_numpy(rng.standard_normal(64 * (n + 8) + 8).astype(np.float32)).cuda()
    base = flat[:64 * (n + 8)].reshape(64, n + 8)
    say("[select many rows] stride n + 8, 64 rows")
    idx, _ = m.topk_select(base, 1000, row_len=n, row_stride=n + 8)
    assert np.array_equal(idx.cpu().numpy(), orc.select(base.cpu().numpy()[:, :n].copy(), 1000))
    say("[select many rows] rows 4 bytes off alignment")
    view = flat[1:1 + 64 * (n + 8)].reshape(64, n + 8)
    idx, _ = m.topk_select(view, 1000, row_len=n, row_stride=n + 8)
    assert np.array_equal(idx.cpu().numpy(), orc.select(view.cpu().numpy()[:, :n].copy(), 1000))
