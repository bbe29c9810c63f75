"""Pins of the producer-op references (oracle/producer.py) against closed
forms, identities and an independent library routine (CPU)."""

import math

import numpy as np
import pytest
from scipy.special import expit

import oracle
import workloads


def _bits(x):
    return workloads.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_rmsnorm_constant_rows_closed_form():
    # a row of one value c: mean(x^2) = c^2, so y = c / sqrt(c^2 + eps) * g
    K, eps = 64, 1e-5
    g = np.linspace(-2, 2, K).astype(np.float32)
    gb = _bits(g)
    gv = workloads.bf16_bits_to_f32(gb).astype(np.float64)
    for c in (1.0, -3.0, 0.015625, 1024.0):
        y = oracle.rmsnorm_ref(_bits(np.full((1, K), c)), gb, eps)
        assert np.allclose(y[0], c / math.sqrt(c * c + eps) * gv, rtol=1e-15, atol=0)


def test_rmsnorm_matches_exact_sums_and_is_scale_free():
    rng = np.random.default_rng(3)
    x = _bits(rng.standard_normal((3, 48)) * 5)
    g = _bits(rng.standard_normal(48))
    xv, gv = workloads.bf16_bits_to_f32(x), workloads.bf16_bits_to_f32(g)
    y = oracle.rmsnorm_ref(x, g, 0.0)
    for m in range(3):
        ms = math.fsum(float(v) * float(v) for v in xv[m]) / 48
        want = [float(xv[m, k]) / math.sqrt(ms) * float(gv[k]) for k in range(48)]
        assert np.allclose(y[m], want, rtol=1e-14, atol=0)
        # with eps = 0 the normalised row has mean square 1 (before the gain)
        assert math.isclose(math.fsum((y[m] / gv) ** 2) / 48, 1.0, rel_tol=1e-12)
    # scaling a row by a power of two leaves the output unchanged (eps = 0)
    y2 = oracle.rmsnorm_ref(_bits(workloads.bf16_bits_to_f32(x) * 8), g, 0.0)
    assert np.array_equal(y, y2)


def test_silu_against_the_logistic_function():
    a = np.concatenate([np.linspace(-30, 30, 601), [0.0, 1e-30, -1e-30, 88.0, -88.0, -700.0]])
    assert np.allclose(oracle.silu_ref(a), a * expit(a), rtol=1e-14, atol=1e-300)
    assert oracle.silu_ref(np.array([0.0]))[0] == 0.0
    # silu(-a) = silu(a) - a
    b = np.linspace(-20, 20, 401)
    assert np.allclose(oracle.silu_ref(-b), oracle.silu_ref(b) - b, rtol=1e-12, atol=1e-12)


def test_swiglu_is_silu_times_up():
    rng = np.random.default_rng(4)
    a = _bits(rng.standard_normal((5, 32)) * 4)
    b = _bits(rng.standard_normal((5, 32)))
    av, bv = workloads.bf16_bits_to_f32(a).astype(np.float64), workloads.bf16_bits_to_f32(b).astype(np.float64)
    assert np.allclose(oracle.swiglu_ref(a, b), av * expit(av) * bv, rtol=1e-14, atol=1e-300)
    ones = _bits(np.ones((5, 32)))
    assert np.allclose(oracle.swiglu_ref(a, ones), av * expit(av), rtol=1e-14, atol=1e-300)
    assert np.all(oracle.swiglu_ref(_bits(np.zeros((2, 8))), b[:2, :8]) == 0)
