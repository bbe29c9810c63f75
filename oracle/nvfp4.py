"""NVFP4 two-level block quantization, written as plainly as possible.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The method ([GS-EN] s.2 Methodology, Hybrid Precision Strategy; the same
passage in [GS-ES] s.2 "Estrategia de precision hibrida") puts weights and
activations of the prefill linears in NVFP4: a local scale for every group of
16 consecutive elements, a tensor-level scale on top, and plain
round-to-nearest for the elements.  The pages name no bit formats; the
readings taken here are:

* element: OCP E2M1 (1 sign, 2 exponent, 1 mantissa bit), magnitudes
  {0, 0.5, 1, 1.5, 2, 3, 4, 6}; a 4-bit code is sign<<3 | magnitude index;
* group ("block") scale: OCP E4M3 "fn" byte (bias 7, largest finite 448,
  0x7F/0xFF are NaN and never produced, subnormals kept);
* tensor scale: one IEEE binary32 value, stored as the *decode* factor
  s_t = amax / (6 * 448), so the largest group scale lands on E4M3's largest
  finite value; 1.0 when the tensor is all zeros;
* "tensor" for an activation is the whole input of one GEMM call, taken at
  run time (no calibration: the pages use plain RTN with nothing fitted);
* round-to-nearest breaks ties to the even code, for elements and for group
  scales alike, and saturates at the largest finite value;
* every scale step is one correctly rounded binary32 operation, in this
  order: rho = (a / 6) / s_t, S = E4M3(rho), d = value(S) * s_t,
  e = 1 / d (0 when d == 0), y = x * e, code = E2M1(|y|) with the sign of x;
* an element whose y is NaN (only x = +-0 times e = +inf, when d is so small
  that 1/d overflows) gets magnitude 0; y = +-inf saturates to 6;
* layout: codes [rows][cols/2] bytes, the even column in the low nibble;
  scales [rows][cols/16] bytes; both row-major.

Inputs are bfloat16 values held in float32 arrays (or raw bf16 bit patterns
as uint16); every binary32 step below is a NumPy float32 operation, which is
IEEE-754 round-to-nearest-even with no FMA contraction and no flush to zero.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# E2M1 magnitudes, indexed by the 3-bit magnitude code (OCP E2M1 layout).
E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
E2M1_MAX = 6.0
E4M3_MAX = 448.0
# 6 * 448: maps the tensor's absolute maximum onto the largest group scale.
TENSOR_SCALE_DIVISOR = np.float32(E2M1_MAX * E4M3_MAX)

GROUP = 16  # elements per local scale ([GS-EN] s.2 Hybrid Precision Strategy)


# ---------------------------------------------------------------------------
# format helpers
# ---------------------------------------------------------------------------

def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen raw bfloat16 bit patterns (uint16) to float32 (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _as_bf16_valued_f32(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x)
    x = x.astype(np.float32, copy=False)
    low = x.view(np.uint32) & np.uint32(0xFFFF)
    if np.any(low):
        raise ValueError("input is not bfloat16-valued")
    if not np.all(np.isfinite(x)):
        raise ValueError("NaN/Inf inputs are outside the quantizer's contract")
    return x


def e4m3_decode(code) -> np.ndarray:
    """Value of an OCP E4M3 'fn' byte as float32 (exact).

    E = code>>3 (bias 7), m = code&7.  E == 0 is subnormal: m * 2^-9.
    0x7F and 0xFF are NaN.  The sign bit is honoured although the quantizer
    only ever produces non-negative scales.
    """
    c = np.asarray(code).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(E == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(E - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return (sign * mag).astype(np.float32)


def e4m3_finite_values():
    """The 127 finite non-negative E4M3 values, ascending, with their codes."""
    codes = np.arange(0x7F, dtype=np.int64)  # 0x00 .. 0x7E
    return e4m3_decode(codes).astype(np.float64), codes


def _nearest_ties_to_even_code(t: np.ndarray, values: np.ndarray,
                               codes: np.ndarray) -> np.ndarray:
    """Code of the value nearest to each t (t >= 0, finite or +inf).

    ``values`` ascending; a t above the largest value maps to the largest
    (saturation); a t exactly halfway between two neighbours takes the one
    whose code is even.  The differences are taken in float64, where they are
    exact whenever two candidates are close enough to compete.
    """
    t = np.asarray(t, dtype=np.float64)
    n = len(values)
    i = np.searchsorted(values, t, side="left")  # values[i-1] < t <= values[i]
    hi = np.clip(i, 0, n - 1)
    lo = np.clip(i - 1, 0, n - 1)
    with np.errstate(invalid="ignore"):
        d_lo = t - values[lo]
        d_hi = values[hi] - t
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    return np.where(take_hi, codes[hi], codes[lo])


def e4m3_encode(rho) -> np.ndarray:
    """Round a non-negative binary32 value to the nearest E4M3 byte.

    Nearest of the 127 finite non-negative values, ties to the even code,
    saturating at 448 (code 0x7E); subnormals (multiples of 2^-9 below 2^-6)
    are kept, so rho <= 2^-10 gives 0.
    """
    rho = np.asarray(rho, dtype=np.float32)
    if np.any(rho < 0) or np.any(np.isnan(rho)):
        raise ValueError("group scale argument must be >= 0 and not NaN")
    values, codes = e4m3_finite_values()
    return _nearest_ties_to_even_code(rho, values, codes).astype(np.uint8)


def e2m1_encode_magnitude(t) -> np.ndarray:
    """3-bit E2M1 magnitude code of |y| (t = |y| as binary32).

    Nearest grid point, ties to the even code, saturating at 6.0; NaN -> 0.
    """
    t = np.asarray(t, dtype=np.float32)
    values = np.asarray(E2M1_GRID, dtype=np.float64)
    codes = np.arange(8, dtype=np.int64)
    nan = np.isnan(t)
    mag = _nearest_ties_to_even_code(np.where(nan, 0.0, np.abs(t)), values, codes)
    return np.where(nan, 0, mag).astype(np.uint8)


def e2m1_decode(code4) -> np.ndarray:
    """Value of 4-bit E2M1 codes (sign<<3 | magnitude) as float64."""
    c = np.asarray(code4).astype(np.int64)
    mag = np.asarray(E2M1_GRID, dtype=np.float64)[c & 7]
    return np.where(c & 8, -mag, mag)


def pack_codes(codes4: np.ndarray) -> np.ndarray:
    """[R][K] 4-bit codes -> [R][K/2] bytes, even column in the low nibble."""
    c = np.asarray(codes4, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """[R][K/2] bytes -> [R][K] 4-bit codes."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# ---------------------------------------------------------------------------
# the quantizer
# ---------------------------------------------------------------------------

@dataclass
class NVFP4Tensor:
    codes: np.ndarray   # uint8 [R][K/2]
    scales: np.ndarray  # uint8 [R][K/16], E4M3 bytes
    s_t: np.float32     # tensor (decode) scale
    amax: np.float32    # max |x| the scale was taken from (0 if given)

    @property
    def shape(self):
        return (self.codes.shape[0], self.codes.shape[1] * 2)


def tensor_scale(amax) -> np.float32:
    """s_t = binary32(amax / 2688), or 1.0 for an all-zero tensor.

    The tensor-level scale of [GS-EN] s.2 Hybrid Precision Strategy, chosen
    so that the group holding the tensor's absolute maximum gets the largest
    finite E4M3 scale.
    """
    a = np.float32(amax)
    if a > 0:
        return np.float32(a / TENSOR_SCALE_DIVISOR)
    return np.float32(1.0)


def quantize_nvfp4(x, s_t=None, rows=None) -> NVFP4Tensor:
    """Quantize a bf16 matrix [R][K] (K % 16 == 0) to NVFP4.

    Steps, in the pages' order (tensor scale, then the per-16 local scale,
    then round-to-nearest of each element; [GS-EN] s.2 Hybrid Precision
    Strategy):

    1. A   = max |x| over the whole tensor (exact).
    2. s_t = binary32(A / 2688), or 1 if A == 0 (unless ``s_t`` is given).
    3. per group of 16 along K: a = max |group|,
       rho = binary32(binary32(a / 6) / s_t), S = E4M3(rho), sigma = value(S).
    4. d = binary32(sigma * s_t); e = binary32(1 / d), or 0 if d == 0.
    5. per element: y = binary32(x * e); code = signbit(x)<<3 | E2M1(|y|).
    6. pack two codes per byte (even column low).

    ``rows``: optional row indices; only those rows are encoded (the tensor
    scale still comes from the whole tensor), so that huge inputs can be
    checked on a sample.
    """
    x = _as_bf16_valued_f32(x)
    if x.ndim != 2 or x.shape[1] % GROUP != 0:
        raise ValueError("expected a [rows][cols] matrix with cols % 16 == 0")
    if s_t is None:
        amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
        s_t = tensor_scale(amax)
    else:
        amax = np.float32(0)
        s_t = np.float32(s_t)
        if not (np.isfinite(s_t) and s_t > 0):
            raise ValueError("a given tensor scale must be finite and > 0")
    if rows is not None:
        x = x[np.asarray(rows)]
    R, K = x.shape
    codes = np.empty((R, K // 2), dtype=np.uint8)
    scales = np.empty((R, K // GROUP), dtype=np.uint8)
    chunk = max(1, (1 << 22) // max(K, 1))  # rows per chunk, bounds temporaries
    six = np.float32(E2M1_MAX)
    one = np.float32(1.0)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore", under="ignore"):
        for r0 in range(0, R, chunk):
            xb = x[r0:r0 + chunk].reshape(-1, K // GROUP, GROUP)
            a = np.max(np.abs(xb), axis=2)                      # float32
            rho = (a / six) / s_t                               # two binary32 divides
            S = e4m3_encode(rho)
            sigma = e4m3_decode(S)
            d = sigma * s_t                                     # binary32 multiply
            e = np.where(d > 0, one / np.where(d > 0, d, one), np.float32(0))
            e = e.astype(np.float32)
            y = xb * e[..., None]                               # binary32 multiply
            mag = e2m1_encode_magnitude(np.abs(y))
            sign = np.signbit(xb).astype(np.uint8)
            c4 = (sign << 3) | mag
            codes[r0:r0 + chunk] = pack_codes(c4.reshape(-1, K))
            scales[r0:r0 + chunk] = S
    return NVFP4Tensor(codes=codes, scales=scales, s_t=np.float32(s_t), amax=amax)


def dequantize_nvfp4(q: NVFP4Tensor, include_tensor_scale: bool = True) -> np.ndarray:
    """x_hat = sign * G[mag] * sigma * s_t as float64 (exact: 6 + 24 bits).

    With ``include_tensor_scale=False`` the s_t factor is left out, giving
    the group-scaled grid values g * sigma.
    """
    c4 = unpack_codes(q.codes)
    R, K = c4.shape
    g = e2m1_decode(c4).reshape(R, K // GROUP, GROUP)
    sigma = e4m3_decode(q.scales).astype(np.float64)
    out = (g * sigma[..., None]).reshape(R, K)
    if include_tensor_scale:
        out = out * np.float64(q.s_t)
    return out
