"""Pins of the oracle quantizer (CPU).

Hand-derived worked examples, the exact round-to-nearest property checked in
exact rationals, and the invariants the two-level scaling must satisfy
(tensor maximum, sign symmetry, power-of-two covariance, permutation within a
group, values already on the grid, idempotence on normal-scale tensors).
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from tests import golden_io
from tests.exact import (e2m1_all_nonneg, e4m3_all_finite_nonneg, f32_exact,
                         nearest_code)


def _bf16(x):
    return workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(np.asarray(x, np.float32)))


@pytest.mark.parametrize("name", golden_io.names())
def test_golden_examples(name):
    g = golden_io.load(name)
    q = oracle.quantize_nvfp4(g["x"])
    assert np.float32(q.s_t).view(np.uint32) == g["s_t_bits"]
    assert np.array_equal(q.scales, g["scales"])
    assert np.array_equal(q.codes, g["codes"])


def test_golden_examples_exist():
    assert len(golden_io.names()) >= 2


def _check_rtn_exact(x, q):
    """Every code is the exact nearest grid point to x / (sigma * s_t) and
    every group scale the exact nearest E4M3 value to a / (6 s_t), except
    where the exact quotient sits within 2^-20 (relative) of a midpoint, where
    the binary32 rounding of the steps legitimately decides."""
    e2 = e2m1_all_nonneg()
    e4 = e4m3_all_finite_nonneg()
    R, K = x.shape
    c4 = oracle.unpack_codes(q.codes)
    s_t = f32_exact(q.s_t)
    A = max(abs(Fraction(float(v))) for v in x.reshape(-1))
    if A > 0:
        # s_t is the binary32 value nearest to A / 2688
        exact = A / 2688
        assert abs(s_t - exact) <= abs(exact) * Fraction(1, 2 ** 24)
    tol = Fraction(1, 2 ** 20)
    e4_mids = [(a + b) / 2 for (_, a), (_, b) in zip(e4[:-1], e4[1:])]
    e2_mids = [(a + b) / 2 for (_, a), (_, b) in zip(e2[:-1], e2[1:])]
    near_mid = lambda v, mids: any(abs(v - m) <= tol * m for m in mids)
    for r in range(R):
        for b in range(K // 16):
            grp = [Fraction(float(v)) for v in x[r, 16 * b:16 * b + 16]]
            a = max(abs(v) for v in grp)
            rho = a / 6 / s_t
            S = int(q.scales[r, b])
            if not near_mid(rho, e4_mids):
                assert S == nearest_code(min(rho, Fraction(448)), e4), (r, b)
            sigma = Fraction(float(oracle.e4m3_decode(np.uint8(S))))
            for j, v in enumerate(grp):
                code = int(c4[r, 16 * b + j])
                assert (code >> 3) == int(np.signbit(x[r, 16 * b + j]))
                if sigma == 0:
                    assert code & 7 == 0
                    continue
                t = abs(v) / (sigma * s_t)
                if not near_mid(t, e2_mids):
                    assert code & 7 == nearest_code(t, e2), (r, b, j, float(t))


@pytest.mark.parametrize("kind,scale,seed", [
    ("normal", 1.0, 0), ("uniform", 3.0, 1), ("lognormal_mixed", 1.0, 2),
    ("normal", 1e-30, 3), ("normal", 1e30, 4),
])
def test_round_to_nearest_exact(kind, scale, seed):
    x = workloads.bf16_bits_to_f32(workloads.random_bf16((3, 64), seed, scale, kind))
    q = oracle.quantize_nvfp4(x)
    _check_rtn_exact(x, q)


def test_round_to_nearest_outliers_cfg1_rows():
    x = workloads.bf16_bits_to_f32(workloads.activation(1))[:2]
    # keep the full tensor's scale: quantize all, check two rows
    full = workloads.bf16_bits_to_f32(workloads.activation(1))
    q = oracle.quantize_nvfp4(full, rows=[0, 1])
    _check_rtn_exact_with_scale(x, q)


def _check_rtn_exact_with_scale(x, q):
    # same as _check_rtn_exact without the s_t-from-these-rows check
    e2 = e2m1_all_nonneg()
    c4 = oracle.unpack_codes(q.codes)
    s_t = f32_exact(q.s_t)
    tol = Fraction(1, 2 ** 20)
    e2_mids = [(a + b) / 2 for (_, a), (_, b) in zip(e2[:-1], e2[1:])]
    for r in range(x.shape[0]):
        for b in range(x.shape[1] // 16):
            sigma = Fraction(float(oracle.e4m3_decode(q.scales[r, b])))
            for j in range(16):
                v = Fraction(float(x[r, 16 * b + j]))
                code = int(c4[r, 16 * b + j])
                if sigma == 0:
                    continue
                t = abs(v) / (sigma * s_t)
                if not any(abs(t - m) <= tol * m for m in e2_mids):
                    assert code & 7 == nearest_code(t, e2)


def test_tensor_max_gets_top_code_and_top_scale():
    x = workloads.bf16_bits_to_f32(workloads.random_bf16((64, 256), 11))
    q = oracle.quantize_nvfp4(x)
    r, k = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    c4 = oracle.unpack_codes(q.codes)
    assert c4[r, k] & 7 == 7
    assert q.scales[r, k // 16] == 0x7E
    assert q.scales.max() == 0x7E


def test_sign_symmetry():
    x = workloads.bf16_bits_to_f32(workloads.random_bf16((32, 128), 12))
    q1 = oracle.quantize_nvfp4(x)
    q2 = oracle.quantize_nvfp4(-x)
    assert np.array_equal(q2.codes, q1.codes ^ 0x88)
    assert np.array_equal(q2.scales, q1.scales)
    assert q1.s_t == q2.s_t


@pytest.mark.parametrize("j", [-20, -3, 1, 7, 30])
def test_power_of_two_covariance(j):
    x = workloads.bf16_bits_to_f32(workloads.random_bf16((16, 128), 13))
    q1 = oracle.quantize_nvfp4(x)
    q2 = oracle.quantize_nvfp4(x * np.float32(2.0 ** j))
    assert np.array_equal(q1.codes, q2.codes)
    assert np.array_equal(q1.scales, q2.scales)
    assert np.float32(q2.s_t) == np.float32(q1.s_t * np.float32(2.0 ** j))


def test_permutation_within_group():
    rng = np.random.default_rng(14)
    x = workloads.bf16_bits_to_f32(workloads.random_bf16((8, 64), 14))
    perm = rng.permutation(16)
    xp = x.reshape(8, 4, 16)[:, :, perm].reshape(8, 64)
    q1, q2 = oracle.quantize_nvfp4(x), oracle.quantize_nvfp4(xp)
    c1 = oracle.unpack_codes(q1.codes).reshape(8, 4, 16)[:, :, perm].reshape(8, 64)
    assert np.array_equal(oracle.unpack_codes(q2.codes), c1)
    assert np.array_equal(q1.scales, q2.scales)


def _on_grid_tensor(rows, cols, j, seed, subnormal_scales=False):
    """x = +-g * sigma * 2^j per group, one group holding 2688 * 2^j."""
    rng = np.random.default_rng(seed)
    vals, codes = oracle.e4m3_finite_values()
    lo = 1 if subnormal_scales else 8
    sig = vals[rng.integers(lo, 0x7F, size=(rows, cols // 16))]
    sig[0, 0] = 448.0
    g = np.asarray(oracle.E2M1_GRID)[rng.integers(0, 8, size=(rows, cols))]
    g = g.reshape(rows, cols // 16, 16)
    g[..., 0] = 6.0  # each group's maximum sits on 6 * sigma
    sign = np.where(rng.random(g.shape) < 0.5, -1.0, 1.0)
    x = (sign * g * sig[..., None]).reshape(rows, cols) * 2.0 ** j
    x32 = x.astype(np.float32)
    assert np.array_equal(x32.astype(np.float64), x)
    assert np.array_equal(_bf16(x32), x32)
    return x32


@pytest.mark.parametrize("j,sub", [(0, False), (-8, False), (5, True), (-3, True)])
def test_values_on_grid_are_exact(j, sub):
    x = _on_grid_tensor(8, 128, j, 15 + j, sub)
    q = oracle.quantize_nvfp4(x)
    assert q.s_t == np.float32(2.0 ** j)
    xh = oracle.dequantize_nvfp4(q)
    assert np.array_equal(np.abs(xh), np.abs(x.astype(np.float64)))
    assert np.array_equal(np.signbit(xh[x != 0]), np.signbit(x[x != 0]))


def test_idempotent_on_normal_scale_tensors():
    x = workloads.bf16_bits_to_f32(workloads.random_bf16((32, 256), 16))
    j = -3
    x[5, 7] = np.float32(2688 * 2.0 ** j)  # makes s_t exactly 2^j
    x = np.clip(x, -2688 * 2.0 ** j, 2688 * 2.0 ** j).astype(np.float32)
    q1 = oracle.quantize_nvfp4(x)
    assert q1.s_t == np.float32(2.0 ** j)
    assert q1.scales.min() >= 0x08  # every group scale is normal
    xh = oracle.dequantize_nvfp4(q1).astype(np.float32)
    assert np.array_equal(_bf16(xh), xh)
    q2 = oracle.quantize_nvfp4(xh)
    assert np.array_equal(q1.codes, q2.codes)
    assert np.array_equal(q1.scales, q2.scales)
    assert q1.s_t == q2.s_t


def test_idempotence_fails_for_subnormal_scale_as_documented():
    # a group with a subnormal scale can re-quantize differently: 0.0187988
    # gets S=0x02 and code 4.0, its dequantized value re-quantizes to S=0x01
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 2688.0
    x[0, 16] = np.float32(0.018798828125)
    q1 = oracle.quantize_nvfp4(x)
    assert q1.scales[0, 1] == 0x02
    xh = oracle.dequantize_nvfp4(q1).astype(np.float32)
    q2 = oracle.quantize_nvfp4(xh)
    assert q2.scales[0, 1] == 0x01
    assert oracle.dequantize_nvfp4(q2)[0, 16] != xh[0, 16]


def test_zero_tensor():
    x = np.zeros((4, 32), np.float32)
    x[1, 3] = -0.0
    q = oracle.quantize_nvfp4(x)
    assert q.s_t == 1.0
    assert np.all(q.scales == 0)
    c4 = oracle.unpack_codes(q.codes)
    assert c4[1, 3] == 8 and np.count_nonzero(c4) == 1


def test_zero_group_in_nonzero_tensor_keeps_sign_only():
    x = workloads.bf16_bits_to_f32(workloads.random_bf16((2, 48), 17))
    x[0, 16:32] = 0.0
    x[0, 20] = -0.0
    x[1, 0:16] = _bf16(np.float32(1e-30))  # far below 2^-10 of the group-scale range
    q = oracle.quantize_nvfp4(x)
    assert q.scales[0, 1] == 0 and q.scales[1, 0] == 0
    c4 = oracle.unpack_codes(q.codes)
    assert np.all(c4[0, 16:32] == np.where(np.arange(16) == 4, 8, 0))
    assert np.all(c4[1, 0:16] == 0)


def test_tiny_tensor_scale_defined_behaviour():
    # amax near the bottom of bf16: s_t is a binary32 subnormal and 1/d can
    # overflow; zeros must still map to magnitude 0 and the run must not raise
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = workloads.bf16_bits_to_f32(np.array([0x0001], np.uint16))[0]  # 2^-133
    x[0, 1] = -x[0, 0]
    x[0, 17] = x[0, 0]
    q = oracle.quantize_nvfp4(x)
    c4 = oracle.unpack_codes(q.codes)
    assert c4[0, 2] == 0 and c4[0, 16] == 0
    assert c4[0, 1] >> 3 == 1 and c4[0, 0] >> 3 == 0
    assert np.all(c4 < 16)


def test_rows_subset_matches_full():
    x = workloads.bf16_bits_to_f32(workloads.random_bf16((40, 96), 18))
    q = oracle.quantize_nvfp4(x)
    rows = [0, 7, 39, 12]
    qs = oracle.quantize_nvfp4(x, rows=rows)
    assert np.array_equal(qs.codes, q.codes[rows])
    assert np.array_equal(qs.scales, q.scales[rows])
    assert qs.s_t == q.s_t


def test_given_scale():
    x = workloads.bf16_bits_to_f32(workloads.random_bf16((4, 32), 19))
    q = oracle.quantize_nvfp4(x, s_t=np.float32(0.5))
    assert q.s_t == np.float32(0.5)
    _check_rtn_exact_with_scale(x, q)


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.quantize_nvfp4(np.zeros((2, 17), np.float32))
    with pytest.raises(ValueError):
        oracle.quantize_nvfp4(np.full((1, 16), 1.0000001, np.float32))
    with pytest.raises(ValueError):
        oracle.quantize_nvfp4(np.full((1, 16), np.inf, np.float32))
