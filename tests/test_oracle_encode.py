"""Pins of the oracle's OCP E4M3FN encoder (the stored form of appended
indexer keys): code values round-trip, midpoints go to the even code, torch's
float8_e4m3fn conversion agrees below 448, values at or above 448 saturate,
NaN encodes as 0x7f, signs (also of zero) are kept."""
import numpy as np
import torch

import fixtures as fx
import oracle as orc

CODES = np.arange(256, dtype=np.uint8)
VALUES = orc.decode_values(fx.E4M3, CODES)
FINITE = CODES[~np.isnan(VALUES)]


def test_every_code_encodes_to_itself():
    v = orc.decode_values(fx.E4M3, FINITE).astype(np.float32)
    got = orc.encode_e4m3(v)
    assert np.array_equal(got, FINITE)


def test_midpoints_round_to_the_even_code():
    pos = np.arange(0, 0x7e, dtype=np.uint8)  # consecutive non-negative codes c, c + 1
    lo = orc.decode_values(fx.E4M3, pos)
    hi = orc.decode_values(fx.E4M3, pos + 1)
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.all(mid.astype(np.float64) == (lo + hi) / 2)  # midpoints are exact in fp32
    got = orc.encode_e4m3(mid)
    want = np.where(pos % 2 == 0, pos, pos + 1).astype(np.uint8)
    assert np.array_equal(got, want)
    assert np.array_equal(orc.encode_e4m3(-mid), want | 0x80)
    # just off the midpoint: the nearer code
    up = np.nextafter(mid, np.float32(np.inf))
    assert np.array_equal(orc.encode_e4m3(up), (pos + 1).astype(np.uint8))


def test_agrees_with_torch_below_448():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.normal(size=20000) * s for s in (0.001, 0.05, 1, 30, 150)]).astype(np.float32)
    x = x[np.abs(x) < 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.encode_e4m3(x), ref)
    assert np.array_equal(orc.encode_e4m3(x), fx.encode(x, fx.E4M3))


def test_saturation_nan_and_signed_zero():
    big = np.array([448, 449, 463.9, 464, 480, 1e6, np.inf], np.float32)
    assert np.all(orc.encode_e4m3(big) == 0x7e) and np.all(orc.encode_e4m3(-big) == 0xfe)
    assert orc.encode_e4m3(np.array([np.nan], np.float32))[0] == 0x7f
    assert list(orc.encode_e4m3(np.array([0.0, -0.0], np.float32))) == [0x00, 0x80]
    tiny = np.array([2.0 ** -12, 2.0 ** -10, 2.0 ** -10 * 1.001], np.float32)
    assert list(orc.encode_e4m3(tiny)) == [0, 0, 1]  # below half the least subnormal, at it (tie to 0), above
