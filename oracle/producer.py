"""Reference definitions of the two ops whose outputs feed the prefill
linears of an 8B-shaped decoder layer: RMSNorm (its output is the input of
the q/k/v and of the gate/up projections) and the SwiGLU gate (its output is
the input of the down projection).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages fix the prefill linears' format (NVFP4 activations with a
tensor-level scale taken at run time, [GS-EN] s.2 Hybrid Precision Strategy)
and name the Llama-style models the method runs on ([GS-EN] s.4
Experimental Results); they do not define these ops.  They enter because a
producer that emits the activation's partial maxima spares the quantizer
its first pass over the activation.  The definitions are the textbook ones
of that layer, written out in float64 from the bf16 inputs:

  RMSNorm       y = x / sqrt(mean_k(x_k^2) + eps) * g        (per row)
  SwiGLU gate   y = silu(a) * b,  silu(a) = a / (1 + exp(-a))

The kernels compute in binary32 and round to bfloat16, so their outputs
differ from these by rounding and are compared with a tolerance; the partial
maxima they emit are checked exactly against their own outputs, and the
quantization of those outputs against ``quantize_nvfp4``.
"""

from __future__ import annotations

import numpy as np


def _bf16_to_f64(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rmsnorm_ref(x_bits, g_bits, eps: float) -> np.ndarray:
    """y[m, k] = x[m, k] / sqrt(mean_k x[m, k]^2 + eps) * g[k], float64."""
    x = _bf16_to_f64(x_bits)
    g = _bf16_to_f64(g_bits).reshape(1, -1)
    ms = np.mean(x * x, axis=1, keepdims=True)
    return x / np.sqrt(ms + np.float64(eps)) * g


def silu_ref(a) -> np.ndarray:
    """silu(a) = a / (1 + exp(-a)) in float64 (a as float64 values)."""
    a = np.asarray(a, dtype=np.float64)
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def swiglu_ref(a_bits, b_bits) -> np.ndarray:
    """y = silu(a) * b elementwise, float64, from bf16 bit patterns."""
    return silu_ref(_bf16_to_f64(a_bits)) * _bf16_to_f64(b_bits)
