"""The division identity the GEMM's fused prologue relies on.

For binary32 x and y != 0, rounding the binary64 product x * RN64(1/y) to
binary32 gives the correctly rounded binary32 quotient RN32(x / y): a
binary32 quotient that is not representable lies at least about 2^-48 of its
size away from every binary32 rounding midpoint (x - M*y is a non-zero
multiple of a fine power of two), while the binary64 product is within
2^-52 of it; and the quotient is a midpoint only when y is a power of two,
where the product is exact.  The fused prologue computes the group scale's
two divisions (a / 6 and (a/6) / s_t) this way.  Checked here against
numpy's binary32 division (IEEE, correctly rounded): exhaustively for a / 6
over every finite bf16 magnitude, and on a large sample, powers of two and
subnormals included, for the division by the tensor scale.
"""

import numpy as np


def _via_reciprocal(x32, y32):
    inv = np.float64(1.0) / y32.astype(np.float64)          # RN64(1/y)
    return (x32.astype(np.float64) * inv).astype(np.float32)  # RN32(RN64(x * inv))


def test_division_by_six_all_bf16_magnitudes():
    bits = np.arange(0, 0x7F80, dtype=np.uint32) << 16       # +0 .. largest finite bf16
    a = bits.view(np.float32)
    six = np.full_like(a, 6.0)
    with np.errstate(all="ignore"):
        exact = a / six
        fast = _via_reciprocal(a, six)
    assert np.array_equal(exact.view(np.uint32), fast.view(np.uint32))


def test_division_by_tensor_scale_sample():
    rng = np.random.default_rng(20261203)
    n = 2_000_000
    # numerators: quotients a/6 of bf16 magnitudes (what the prologue divides)
    a = (rng.integers(0, 0x7F80, n, dtype=np.uint32) << 16).view(np.float32)
    x = (a / np.float32(6.0)).astype(np.float32)
    # divisors: positive finite binary32 of every exponent, plus powers of two
    y = rng.integers(1, 0x7F800000, n, dtype=np.uint32).view(np.float32)
    y[: n // 8] = (rng.integers(1, 255, n // 8, dtype=np.uint32) << 23).view(np.float32)
    with np.errstate(all="ignore"):
        exact = x / y
        fast = _via_reciprocal(x, y)
    finite = np.isfinite(exact)
    assert finite.sum() > n // 2
    assert np.array_equal(exact[finite].view(np.uint32), fast[finite].view(np.uint32))


def test_division_midpoint_and_subnormal_cases():
    # quotients exactly on a binary32 midpoint (divisor a power of two) and
    # results in the subnormal range
    x = np.array([3 * 2.0 ** -149, 5 * 2.0 ** -149, 2.0 ** -126, 1.5, 3.0, 1e-38, 7e-45],
                 dtype=np.float64).astype(np.float32)
    for y in np.array([2.0, 4.0, 3.0, 6.0, 1e10, 2688.0, 0.5], dtype=np.float32):
        yy = np.full_like(x, y)
        with np.errstate(all="ignore"):
            assert np.array_equal((x / yy).view(np.uint32), _via_reciprocal(x, yy).view(np.uint32))
