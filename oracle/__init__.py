"""CPU oracle for the NVFP4 prefill linear and the BF16 decode GEMV.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything in this package: only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.  The
HIP library never falls back to it.

It is deliberately plain and slow: NumPy float32 for every step the method
defines in binary32 (each one a single IEEE-754 round-to-nearest-even
operation; NumPy never contracts a multiply and an add into an FMA), and
float64 for the reference contractions.  It shares no code, table or constant
generator with the HIP kernels.

Pages cited, by title and section:

  [GS-EN]  gist.science, English explainer of "Mix-Quant: Quantized
           Prefilling, Precise Decoding for Agentic LLMs", Technical Summary.
  [GS-ES]  gist.science, the Spanish version of the same explainer,
           "Resumen Tecnico".
  [ZX]     zingnex.cn forum digest of the same paper, sections on the
           prefill (FP4) and decode (BF16) stages.

What the pages fix: the prefill linears run with weights and activations both
in NVFP4 ([GS-EN] s.2 System-Level Deployment, "W4A4"); NVFP4 has a local
scale per group of 16 elements plus a tensor-level scale, and elements are
quantized by plain round-to-nearest ([GS-EN] s.2 Hybrid Precision Strategy);
decode keeps the original BF16 weights ([GS-EN] s.2 Hybrid Precision
Strategy, Decoding).  Everything else (element and scale formats, the tensor
scale's value, tie rule, rounding order) is a reading stated in the docstring
of the function that takes it.

Parity status: every function here is pinned by tests under ``tests/`` that
check it against something other than itself (brute force over exact
rationals, torch's float8_e4m3fn cast, closed forms, invariants).  No
function is "parity unpinned".
"""

from .nvfp4 import (  # noqa: F401
    E2M1_GRID,
    E4M3_MAX,
    E2M1_MAX,
    TENSOR_SCALE_DIVISOR,
    e2m1_encode_magnitude,
    e2m1_decode,
    e4m3_encode,
    e4m3_decode,
    e4m3_finite_values,
    tensor_scale,
    quantize_nvfp4,
    dequantize_nvfp4,
    pack_codes,
    unpack_codes,
    NVFP4Tensor,
)
from .linear import (  # noqa: F401
    gemm_nvfp4_ref,
    gemm_nvfp4_ref_rows,
    gemv_bf16_ref,
    round_f64_to_bf16,
)
from .producer import (  # noqa: F401
    rmsnorm_ref,
    silu_ref,
    swiglu_ref,
)
