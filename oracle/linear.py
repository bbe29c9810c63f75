"""Reference contractions for the prefill GEMM and the decode GEMV.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Prefill: the W4A4 linear of [GS-EN] s.2 System-Level Deployment (prefill
workers) multiplies the NVFP4 activations by the NVFP4 weights.  Its plain
definition is the dense product of the two dequantized operands,
C = DQ(A) . DQ(W)^T with W stored [N][K] (no bias), which is what is computed
here, in float64, with NumPy's matmul as the one library step.  The kernel
accumulates in binary32 and rounds to bfloat16, so its result is not unique;
tests compare it with a tolerance.

Decode: [GS-EN] s.2 Hybrid Precision Strategy (Decoding) and System-Level
Deployment (decode workers) keep the original BF16 weights; the reference is
Y = X . W^T on the bf16 values, in float64.
"""

from __future__ import annotations

import numpy as np

from .nvfp4 import NVFP4Tensor, dequantize_nvfp4, unpack_codes, e2m1_decode, e4m3_decode, GROUP


def gemm_nvfp4_ref(a: NVFP4Tensor, w: NVFP4Tensor) -> np.ndarray:
    """C64[m, n] = sum_k DQ(A)[m, k] * DQ(W)[n, k] in float64.

    The group-scaled grid values g*sigma are exact in float64; the tensor
    scales are applied once to the product, C = (s_tA * s_tW) * P.
    """
    if a.shape[1] != w.shape[1]:
        raise ValueError("K mismatch")
    pa = dequantize_nvfp4(a, include_tensor_scale=False)
    pw = dequantize_nvfp4(w, include_tensor_scale=False)
    return (pa @ pw.T) * (np.float64(a.s_t) * np.float64(w.s_t))


def gemm_nvfp4_ref_rows(a: NVFP4Tensor, w: NVFP4Tensor) -> np.ndarray:
    """Same as :func:`gemm_nvfp4_ref`, spelled out group by group.

    C64[m, n] = s_tA * s_tW * sum_b sigmaA[m, b] * sigmaW[n, b]
                * sum_{k in b} gA[m, k] * gW[n, k].
    Slow; meant for a few rows as a cross-check of the matmul form.
    """
    ga = e2m1_decode(unpack_codes(a.codes))
    gw = e2m1_decode(unpack_codes(w.codes))
    sa = e4m3_decode(a.scales).astype(np.float64)
    sw = e4m3_decode(w.scales).astype(np.float64)
    M, K = ga.shape
    N = gw.shape[0]
    nb = K // GROUP
    out = np.zeros((M, N), dtype=np.float64)
    for b in range(nb):
        ks = slice(b * GROUP, (b + 1) * GROUP)
        p = ga[:, ks] @ gw[:, ks].T  # exact: small integers and halves
        out += p * (sa[:, b][:, None] * sw[:, b][None, :])
    return out * (np.float64(a.s_t) * np.float64(w.s_t))


def gemv_bf16_ref(x, w) -> np.ndarray:
    """Y64 = X . W^T on bf16-valued inputs, in float64 (products exact)."""
    x64 = np.asarray(x, dtype=np.float64)
    w64 = np.asarray(w, dtype=np.float64)
    return x64 @ w64.T


def round_f64_to_bf16(v) -> np.ndarray:
    """Round float64 values straight to bfloat16 (nearest, ties to even).

    Rounds once from float64 (rounding through float32 first could round
    twice).  Returns float64 holding bf16 values; overflow gives +-inf.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros_like(v)
    nz = (v != 0) & np.isfinite(v)
    m, e = np.frexp(v[nz])             # v = m * 2^e, 0.5 <= |m| < 1
    q = np.maximum(e - 8, -133)         # bf16 quantum exponent (8 significant bits)
    r = np.rint(np.ldexp(v[nz], -q))    # exact scaling, then round half even
    res = np.ldexp(r, q)
    bf16_max = np.ldexp(np.float64(0xFF), 127 - 7)  # (2 - 2^-7) * 2^127
    res = np.where(np.abs(res) > bf16_max, np.copysign(np.inf, res), res)
    out[nz] = res
    out[~np.isfinite(v)] = v[~np.isfinite(v)]
    return out
