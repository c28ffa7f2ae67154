"""Pins of number decoding (oracle) and encoding (fixtures) against torch's
own bfloat16 and float8_e4m3fn types (OCP E4M3FN: bias 7, max 448, S.1111.111
NaN, no infinities), plus determinism and structure of the seeded inputs."""
import json
import os

import numpy as np
import torch

import fixtures as fx
import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _same(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)])


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert _same(orc.decode_values(orc.E4M3, codes), ref)
    assert orc.decode_values(orc.E4M3, np.array([0x7E], np.uint8))[0] == 448.0


def test_bf16_decode_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same(orc.decode_values(orc.BF16, codes), ref)


def _probe_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 3, 20000),
                        [0.0, -0.0, 1e-40, -1e-40, 3.0e38, np.inf, -np.inf]]).astype(np.float32)
    # exact ties for bf16 rounding
    ties = (np.arange(1000, dtype=np.uint32) * 65536 + 0x3F800000 + 0x8000).view(np.float32)
    return np.concatenate([x, ties])


def test_bf16_encode_matches_torch():
    x = _probe_values()
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(fx.encode(x, fx.BF16), ref)


def test_e4m3_encode_matches_torch_in_range_and_saturates():
    x = _probe_values()
    x = x[np.isfinite(x) & (np.abs(x) < 448)]
    # midpoints between neighbouring codes exercise ties-to-even
    vals = orc.decode_values(orc.E4M3, np.arange(0, 0x7E, dtype=np.uint8))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fx.encode(x, fx.E4M3), ref)
    sat = fx.encode(np.array([448.0, 460.0, 1e6, -1e6, np.inf, -np.inf], np.float32), fx.E4M3)
    assert sat.tolist() == [0x7E, 0x7E, 0x7E, 0xFE, 0x7E, 0xFE]
    assert fx.encode(np.array([np.nan], np.float32), fx.E4M3)[0] == 0x7F


def test_normal_stream_statistics_and_independence():
    z = fx.normal(9, 1, 400000).astype(np.float64)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    # any slice regenerates identically on its own
    assert np.array_equal(fx.normal(9, 1, 1000, offset=12345), z[12345:13345].astype(np.float32))
    assert not np.array_equal(fx.normal(9, 2, 1000), fx.normal(9, 1, 1000))


def test_sample_distinct():
    s = fx.sample_distinct(3, 7, 131072, 655)
    assert len(np.unique(s)) == 655 and np.all(np.diff(s) > 0) and s.min() >= 0 and s.max() < 131072


def test_aligned_plants_have_requested_cosine():
    w = fx.shrink(fx.WORKLOADS["C2"], 4096, B=1)
    q, K, V = fx.make_attn(w)
    qf, Kf = fx.bf16_bits_to_f32(q).astype(np.float64), fx.bf16_bits_to_f32(K).astype(np.float64)
    G = w.Hq // w.Hkv
    for g in range(w.Hkv):
        pos = fx.sample_distinct(w.seed, g, w.L, w.n_plant)
        for j, p in enumerate(pos):
            h = g * G + j % G
            kr, qh = Kf[0, g, p], qf[0, h]
            cos = kr @ qh / np.linalg.norm(kr) / np.linalg.norm(qh)
            assert abs(cos - 0.5) < 0.01


def test_block_shift_moves_block_means_toward_query():
    w = fx.shrink(fx.WORKLOADS["C4"], 64 * 200, B=1)
    q, K, V = fx.make_attn(w)
    qf, Kf = fx.bf16_bits_to_f32(q).astype(np.float64), fx.bf16_bits_to_f32(K).astype(np.float64)
    G = w.Hq // w.Hkv
    blocks = fx.sample_distinct(w.seed, 0, w.m, w.n_plant)
    for j, blk in enumerate(blocks):
        h = j % G
        mu = Kf[0, 0, blk * 64:(blk + 1) * 64].mean(0)
        qh = qf[0, h] / np.linalg.norm(qf[0, h])
        assert abs(mu @ qh - w.plant_param) < 0.5  # mean of 64 N(0,1) projections has sd 1/8


def test_fixture_digests_match_golden():
    with open(os.path.join(GOLDEN, "fixture_digests.json")) as f:
        gold = json.load(f)
    from tests.golden.make_fixture_digests import current_digests
    assert current_digests() == gold
