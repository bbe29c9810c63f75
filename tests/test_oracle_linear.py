"""Pins of the oracle GEMM / GEMV references (CPU).

Exact-rational brute force on tiny shapes, two independent formulations of
the block-scaled product, closed forms that tie the quantizer to the GEMM,
and one-hot probes that expose a transposed or shifted operand.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from tests.exact import f32_exact


def _q(shape, seed, kind="normal", scale=1.0):
    x = workloads.bf16_bits_to_f32(workloads.random_bf16(shape, seed, scale, kind))
    return x, oracle.quantize_nvfp4(x)


def _exact_gemm(a, w):
    """sum_k DQ(A)[m,k] DQ(W)[n,k] in exact rationals, from the bytes."""
    def vals(q):
        c4 = oracle.unpack_codes(q.codes)
        R, K = c4.shape
        g = [0, Fraction(1, 2), 1, Fraction(3, 2), 2, 3, 4, 6]
        out = []
        for r in range(R):
            row = []
            for k in range(K):
                code = int(c4[r, k])
                sig = Fraction(float(oracle.e4m3_decode(q.scales[r, k // 16])))
                v = g[code & 7] * sig * f32_exact(q.s_t)
                row.append(-v if code & 8 else v)
            out.append(row)
        return out
    A, W = vals(a), vals(w)
    return [[sum(x * y for x, y in zip(ra, rw)) for rw in W] for ra in A]


@pytest.mark.parametrize("M,N,K,seed", [(16, 16, 16, 0), (32, 48, 64, 1), (3, 5, 32, 2)])
def test_gemm_matches_exact_rational_brute_force(M, N, K, seed):
    _, a = _q((M, K), seed, "lognormal_mixed")
    _, w = _q((N, K), seed + 100, "normal", 0.02)
    ref = oracle.gemm_nvfp4_ref(a, w)
    ex = _exact_gemm(a, w)
    for m in range(M):
        for n in range(N):
            e = ex[m][n]
            assert abs(Fraction(float(ref[m, n])) - e) <= abs(e) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 1000)


def test_gemm_two_formulations_agree():
    _, a = _q((24, 96), 3, "uniform", 5.0)
    _, w = _q((40, 96), 4, "normal", 0.02)
    r1 = oracle.gemm_nvfp4_ref(a, w)
    r2 = oracle.gemm_nvfp4_ref_rows(a, w)
    assert np.allclose(r1, r2, rtol=1e-13, atol=0)


def test_gemm_identity_weight_closed_form():
    # W = 2688 * I quantizes exactly (s_t = 1, S = 0x7E, code 7 on the
    # diagonal), so C = 2688 * DQ(A): ties the quantizer to the GEMM.
    K = 64
    w = np.eye(K, dtype=np.float32) * np.float32(2688.0)
    qw = oracle.quantize_nvfp4(w)
    assert qw.s_t == 1.0
    diag_group = (np.arange(K) // 16)[:, None] == np.arange(K // 16)[None, :]
    assert np.array_equal(qw.scales, np.where(diag_group, 0x7E, 0).astype(np.uint8))
    assert np.array_equal(oracle.dequantize_nvfp4(qw), w.astype(np.float64))
    x, qa = _q((10, K), 5)
    c = oracle.gemm_nvfp4_ref(qa, qw)
    assert np.array_equal(c, 2688.0 * oracle.dequantize_nvfp4(qa))


def test_gemm_constant_closed_form():
    M, N, K = 7, 9, 48
    a = np.full((M, K), 1.5, np.float32)
    w = np.full((N, K), -0.25, np.float32)
    qa, qw = oracle.quantize_nvfp4(a), oracle.quantize_nvfp4(w)
    da = oracle.dequantize_nvfp4(qa)[0, 0]
    dw = oracle.dequantize_nvfp4(qw)[0, 0]
    c = oracle.gemm_nvfp4_ref(qa, qw)
    assert np.allclose(c, K * da * dw, rtol=1e-15)
    assert abs(da - 1.5) / 1.5 < 0.07 and abs(dw + 0.25) / 0.25 < 0.07


def test_gemm_one_hot_rows_pick_weight_columns():
    # A row m has a single nonzero (the tensor max) at column k_m, so
    # C[m, n] = 2688 * s_tA * DQ(W)[n, k_m] / ... exposes transposes/shifts
    M, N, K = 6, 5, 64
    ks = [0, 17, 33, 63, 8, 40]
    a = np.zeros((M, K), np.float32)
    for m, k in enumerate(ks):
        a[m, k] = 2688.0
    qa = oracle.quantize_nvfp4(a)
    assert np.array_equal(oracle.dequantize_nvfp4(qa), a.astype(np.float64))
    _, qw = _q((N, K), 6)
    c = oracle.gemm_nvfp4_ref(qa, qw)
    dw = oracle.dequantize_nvfp4(qw)
    for m, k in enumerate(ks):
        assert np.array_equal(c[m], 2688.0 * dw[:, k])


def test_gemv_one_hot_and_brute_force():
    N, K = 12, 64
    w = workloads.bf16_bits_to_f32(workloads.random_bf16((N, K), 7))
    x = np.zeros((3, K), np.float32)
    x[0, 5] = 1.0
    x[1, 63] = -2.0
    x[2] = workloads.bf16_bits_to_f32(workloads.random_bf16((K,), 8))
    y = oracle.gemv_bf16_ref(x, w)
    assert np.array_equal(y[0], w[:, 5].astype(np.float64))
    assert np.array_equal(y[1], -2.0 * w[:, 63].astype(np.float64))
    for n in range(N):
        ex = sum(Fraction(float(p)) * Fraction(float(q)) for p, q in zip(x[2], w[n]))
        assert abs(Fraction(float(y[2, n])) - ex) <= abs(ex) * Fraction(1, 2 ** 48) + Fraction(1, 2 ** 900)


def test_rule_t_helper_accepts_truth_and_rejects_planted_error():
    from tests.parity import rule_t
    _, a = _q((32, 128), 9)
    _, w = _q((48, 128), 10, "normal", 0.02)
    ref = oracle.gemm_nvfp4_ref(a, w)
    good = oracle.round_f64_to_bf16(ref)
    assert rule_t(good, ref, bf16_out=True).ok
    assert rule_t(ref.astype(np.float32), ref, bf16_out=False).ok
    # a planted mistake in the reference (one dropped K-group) must fail
    a2 = oracle.NVFP4Tensor(a.codes.copy(), a.scales.copy(), a.s_t, a.amax)
    a2.scales[:, 3] = 0
    bad = oracle.round_f64_to_bf16(oracle.gemm_nvfp4_ref(a2, w))
    assert not rule_t(bad, ref, bf16_out=True).ok
    # a transposed scale product must fail too
    swapped = oracle.round_f64_to_bf16(ref * 1.01)
    assert not rule_t(swapped, ref, bf16_out=True).ok
