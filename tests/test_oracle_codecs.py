"""Pins of the oracle's element and scale codecs (CPU).

E4M3: decode against torch's float8_e4m3fn for all 256 bytes; encode against
exhaustive exact-rational nearest search and against torch's cast.
E2M1: encode against exhaustive exact-rational nearest search on every
bf16 value in range and on float32 values packed around each tie point, and
against the tie table that the nearest-even rule implies.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.exact import (e2m1_all_nonneg, e4m3_all_finite_nonneg, f32_exact,
                         nearest_bf16, nearest_code)
from fractions import Fraction


def _f32_neighbourhood(centres, ulps=4):
    out = []
    for c in centres:
        u = np.float32(c).view(np.uint32).astype(np.int64)
        for d in range(-ulps, ulps + 1):
            if u + d >= 0:
                out.append(np.uint32(u + d))
    return np.array(out, dtype=np.uint32).view(np.float32)


def test_e4m3_decode_matches_torch_all_bytes():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_e4m3_decode_matches_bit_layout():
    table = e4m3_all_finite_nonneg()
    vals = oracle.e4m3_decode(np.array([c for c, _ in table], dtype=np.uint8))
    for (c, v), o in zip(table, vals):
        assert Fraction(float(o)) == v, hex(c)
    assert float(oracle.e4m3_decode(np.uint8(0x7E))) == 448.0
    assert float(oracle.e4m3_decode(np.uint8(0x01))) == 2.0 ** -9


def _e4m3_samples():
    table = e4m3_all_finite_nonneg()
    vals = [v for _, v in table]
    mids = [float((a + b) / 2) for a, b in zip(vals[:-1], vals[1:])]
    t = list(_f32_neighbourhood(mids + [float(v) for v in vals] + [448.0, 464.0, 2.0 ** -10], ulps=3))
    rng = np.random.default_rng(1234)
    t += list((np.exp2(rng.uniform(-12, 9.2, 3000))).astype(np.float32))
    t += [np.float32(0.0), np.float32(1e-30), np.float32(500.0), np.float32(3e38)]
    return np.array(t, dtype=np.float32)


def test_e4m3_encode_matches_exhaustive_exact_search():
    table = e4m3_all_finite_nonneg()
    t = _e4m3_samples()
    ours = oracle.e4m3_encode(t)
    for ti, oi in zip(t, ours):
        assert nearest_code(f32_exact(ti), table) == oi, (float(ti), int(oi))


def test_e4m3_encode_matches_torch_cast_on_every_bf16_and_dense_f32():
    # every non-negative bf16 pattern below 464 plus a dense float32 sweep
    bits = np.arange(0, 0x7F80, dtype=np.uint32) << 16
    t = bits.view(np.float32)
    t = t[t <= 464.0]
    rng = np.random.default_rng(7)
    dense = rng.integers(0, np.float32(464.0).view(np.uint32), 2_000_000, dtype=np.uint32).view(np.float32)
    t = np.concatenate([t, dense])
    ours = oracle.e4m3_encode(t)
    ref = torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_saturates_above_max():
    t = np.array([448.0, 464.0, 465.0, 480.0, 1e5, np.inf], dtype=np.float32)
    assert np.all(oracle.e4m3_encode(t) == 0x7E)


def test_e2m1_tie_table():
    # the seven midpoints and where nearest-even sends them
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for t, code in ties.items():
        assert int(oracle.e2m1_encode_magnitude(np.float32(t))) == code, t
    # just above / below each midpoint goes to the nearer side
    grid = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    for i, mid in enumerate([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]):
        below = np.nextafter(np.float32(mid), np.float32(0))
        above = np.nextafter(np.float32(mid), np.float32(10))
        assert int(oracle.e2m1_encode_magnitude(below)) == i
        assert int(oracle.e2m1_encode_magnitude(above)) == i + 1
    assert grid[-1] == oracle.E2M1_GRID[-1]


def test_e2m1_encode_matches_exhaustive_exact_search():
    table = e2m1_all_nonneg()
    assert [float(v) for _, v in table] == list(oracle.E2M1_GRID)
    # every non-negative bf16 value up to 16, float32 packed around ties,
    # random float32 over many binades
    bits = np.arange(0, 0x4180, dtype=np.uint32) << 16
    t = list(bits.view(np.float32)[::3])
    t += list(_f32_neighbourhood([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.5, 1.0], ulps=6))
    rng = np.random.default_rng(99)
    t += list(np.exp2(rng.uniform(-30, 10, 4000)).astype(np.float32))
    t = np.array(t, dtype=np.float32)
    ours = oracle.e2m1_encode_magnitude(t)
    for ti, oi in zip(t, ours):
        assert nearest_code(f32_exact(ti), table) == oi, float(ti)


def test_e2m1_special_values():
    t = np.array([np.inf, np.nan, 0.0, 1e30, 6.0, 7.0, 1e-45], dtype=np.float32)
    assert list(oracle.e2m1_encode_magnitude(t)) == [7, 0, 0, 7, 7, 7, 0]


def test_e2m1_decode_and_pack_roundtrip():
    codes = np.arange(16, dtype=np.uint8)
    vals = oracle.e2m1_decode(codes)
    assert list(vals[:8]) == list(oracle.E2M1_GRID)
    assert list(vals[8:]) == [-v for v in oracle.E2M1_GRID]
    c = np.random.default_rng(0).integers(0, 16, (5, 32), dtype=np.uint8)
    p = oracle.pack_codes(c)
    assert p.shape == (5, 16)
    assert np.array_equal(p[:, 0], c[:, 0] | (c[:, 1] << 4))   # even column low
    assert np.array_equal(oracle.unpack_codes(p), c)


def test_round_f64_to_bf16_matches_exact_nearest():
    rng = np.random.default_rng(5)
    v = np.concatenate([
        rng.standard_normal(3000) * np.exp2(rng.uniform(-40, 40, 3000)),
        # exact ties: 1 + 2^-8 sits halfway between 1 and 1 + 2^-7
        np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 1 + 2.0 ** -8 + 2.0 ** -40]),
    ])
    ours = oracle.round_f64_to_bf16(v)
    for vi, oi in zip(v, ours):
        assert Fraction(float(oi)) == nearest_bf16(Fraction(float(vi))), vi
    assert oracle.round_f64_to_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert oracle.round_f64_to_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
