"""GPU parity of the producer ops with the amax pass folded in
(mq_rmsnorm_amax, mq_swiglu_amax), and of the RMSNorm fused with the
quantization (mq_rmsnorm_quantize_nvfp4, bit-identical to the producer
followed by the partial-maxima quantization).

Each output is compared element by element with the float64 oracle (within
bf16 rounding of binary32 arithmetic).  The partial maxima they leave in the
scale record must be exactly those of their own stored outputs, and
quantizing the output with MQ_SCALE_PARTIALS (no amax pass) must give the
codes, scales and s_t of the dynamic quantization of that output, which in
turn equal the oracle's quantization bit for bit.
"""

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import announce, quantized_host, to_dev_bf16

pytestmark = pytest.mark.gpu

# bf16 rounding is at most 2^-9 relative; binary32 arithmetic before it adds
# a few 2^-24; silu's hardware exp and reciprocal a few 2^-22
REL_TOL = 2.0 ** -8


def _mq():
    import fp4_block_scaled_elem_amd as mq
    return mq


def _host_bits(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _check_values(y_bits, ref):
    y = workloads.bf16_bits_to_f32(y_bits).astype(np.float64)
    err = np.abs(y - ref)
    bad = err > REL_TOL * np.abs(ref) + 1e-30  # below 1e-30: flush-to-zero of silu's tail is fine
    assert not bad.any(), f"{int(bad.sum())} elements off, worst {np.unravel_index(np.argmax(err - REL_TOL * np.abs(ref)), ref.shape)}"


def _check_partials_and_quantization(y_dev, y_bits, q):
    import torch
    mq = _mq()
    rec = q.rec.cpu().numpy().view(np.uint32)
    nparts = int(rec[2])
    assert 1 <= nparts <= mq.MQ_AMAX_PARTS
    amax_bits = int((y_bits & 0x7FFF).max()) << 16
    assert int(rec[4:4 + nparts].max()) == amax_bits
    # encode alone from the partials vs the dynamic two-pass quantization
    mq.mq_quantize_nvfp4(y_dev, q, mq.MQ_SCALE_PARTIALS)
    c1, s1, t1 = quantized_host(q)
    q2 = mq.quantize(y_dev)
    torch.cuda.synchronize()
    c2, s2, t2 = quantized_host(q2)
    assert t1 == t2 and np.array_equal(s1, s2) and np.array_equal(c1, c2)
    ref = oracle.quantize_nvfp4(y_bits)
    assert t1 == int(np.float32(ref.s_t).view(np.uint32))
    assert np.array_equal(s1, ref.scales) and np.array_equal(c1, ref.codes)


@pytest.mark.parametrize("rows,cols,seed", [(1, 16, 0), (7, 48, 1), (37, 4096, 2), (300, 1040, 3),
                                            (4096, 4096, 4), (3, 14336, 5)])
def test_rmsnorm_amax(rows, cols, seed):
    announce("rmsnorm_amax", rows, cols)
    import torch
    mq = _mq()
    xb = workloads.random_bf16((rows, cols), seed, 1.0, "lognormal_mixed")
    gb = workloads.random_bf16((cols,), seed + 100, 1.0)
    eps = 1e-5
    x, g = to_dev_bf16(xb), to_dev_bf16(gb)
    y = torch.empty_like(x)
    q = mq.NVFP4.empty(rows, cols)
    mq.mq_rmsnorm_amax(x, g, y, q, eps)
    torch.cuda.synchronize()
    yb = _host_bits(y)
    _check_values(yb, oracle.rmsnorm_ref(xb, gb, eps))
    _check_partials_and_quantization(y, yb, q)


@pytest.mark.parametrize("rows,cols,seed", [(1, 16, 0), (5, 48, 1), (64, 14336, 2), (1000, 272, 3),
                                            (4096, 14336, 4)])
def test_swiglu_amax(rows, cols, seed):
    announce("swiglu_amax", rows, cols)
    import torch
    mq = _mq()
    ab = workloads.random_bf16((rows, cols), seed, 4.0)       # gate pre-activations
    bb = workloads.random_bf16((rows, cols), seed + 50, 1.0)  # up projection
    if rows * cols >= 32:
        ab.reshape(-1)[:8] = workloads.f32_to_bf16_bits(np.array([-100, -30, -0.0, 0, 1e-30, 30, 100, -88],
                                                                  np.float32))
    a, b = to_dev_bf16(ab), to_dev_bf16(bb)
    y = torch.empty_like(a)
    q = mq.NVFP4.empty(rows, cols)
    mq.mq_swiglu_amax(a, b, y, q)
    torch.cuda.synchronize()
    yb = _host_bits(y)
    _check_values(yb, oracle.swiglu_ref(ab, bb))
    _check_partials_and_quantization(y, yb, q)


def test_fused_gemm_and_linear_take_the_partials():
    # the GEMM's fused prologue and the phase-aware linear reduce the
    # producer's partial maxima instead of running the amax pass; outputs
    # are bit-identical to the dynamic quantization's
    announce("partials into fused gemm and linear")
    import torch
    mq = _mq()
    M, K, N = 256, 1024, 512
    xb = workloads.random_bf16((M, K), 61, 1.0, "lognormal_mixed")
    gb = workloads.random_bf16((K,), 62, 1.0)
    x, g = to_dev_bf16(xb), to_dev_bf16(gb)
    y = torch.empty_like(x)
    a = mq.NVFP4(None, None, torch.zeros(mq.REC_BYTES // 4, dtype=torch.int32, device="cuda"))
    mq.mq_rmsnorm_amax(x, g, y, a.rec)
    lin = mq.Linear(to_dev_bf16(workloads.random_bf16((N, K), 63, 0.02))).prepare()
    c1 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mq.mq_gemm_nvfp4_prefill(a, y, lin.w_nvfp4, c1, mq.MQ_A_FUSED_BF16 | mq.MQ_SCALE_PARTIALS)
    c2 = mq.prefill_linear(y, lin.w_nvfp4)
    aw = mq.NVFP4.empty(M, K)
    mq.mq_rmsnorm_amax(x, g, y, aw)
    c3 = lin.forward(y, flags=mq.MQ_SCALE_PARTIALS, a_work=aw)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))
    assert torch.equal(c3.view(torch.int16), c2.view(torch.int16))


@pytest.mark.parametrize("rows,cols,seed,gscale", [(1, 16, 10, 1.0), (7, 48, 11, 1.0), (37, 4096, 12, 1.0),
                                                   (300, 1040, 13, 1.0), (4096, 4096, 14, 1.0),
                                                   (3, 14336, 15, 1.0), (2, 4112, 16, 1.0),
                                                   (64, 512, 17, 1.0e-38)])
def test_rmsnorm_quantize_nvfp4(rows, cols, seed, gscale):
    # the RMSNorm fused with quantization (its bf16 output never stored):
    # codes, scales and s_t bit-identical to mq_rmsnorm_amax followed by
    # the partial-maxima quantization, and to the oracle's quantization of
    # that y; rows past 4096 elements (read twice) and odd group counts
    # included, and a gamma near the bottom of bf16's range (y tiny, the
    # tensor scale subnormal: reciprocal group scales overflow, the
    # encoder's fix-up path)
    announce("rmsnorm_quantize_nvfp4", rows, cols, gscale)
    import torch
    mq = _mq()
    xb = workloads.random_bf16((rows, cols), seed, 1.0, "lognormal_mixed")
    gb = workloads.random_bf16((cols,), seed + 100, gscale)
    eps = 1e-5
    x, g = to_dev_bf16(xb), to_dev_bf16(gb)
    q = mq.NVFP4.empty(rows, cols)
    mq.mq_rmsnorm_quantize_nvfp4(x, g, q, eps)
    y = torch.empty_like(x)
    q2 = mq.NVFP4.empty(rows, cols)
    mq.mq_rmsnorm_amax(x, g, y, q2, eps)
    mq.mq_quantize_nvfp4(y, q2, mq.MQ_SCALE_PARTIALS)
    torch.cuda.synchronize()
    c1, s1, t1 = quantized_host(q)
    c2, s2, t2 = quantized_host(q2)
    assert t1 == t2 and np.array_equal(s1, s2) and np.array_equal(c1, c2)
    yb = _host_bits(y)
    ref = oracle.quantize_nvfp4(yb)
    assert t1 == int(np.float32(ref.s_t).view(np.uint32))
    assert np.array_equal(s1, ref.scales) and np.array_equal(c1, ref.codes)
    if gscale >= 1.0e-30:
        _check_values(yb, oracle.rmsnorm_ref(xb, gb, eps))
    else:
        # the fix-up path was taken: some reciprocal group scale overflows
        assert np.float32(ref.s_t) < np.float32(2.0 ** -126)
