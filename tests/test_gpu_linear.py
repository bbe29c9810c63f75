"""GPU parity of the phase-aware linear (mq_linear_prepare / mq_linear_forward).

One weight kept in both formats, each call routed to its phase's path: the
NVFP4 copy made by prepare must equal the oracle's quantization bit for bit,
and each path's output must be bit-identical to the direct calls it stands
for (and within rule T of the float64 oracle).
"""

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import announce, bf16_dev_to_f64, quantized_host, to_dev_bf16
from tests.parity import rule_t

pytestmark = pytest.mark.gpu


def _mq():
    import fp4_block_scaled_elem_amd as mq
    return mq


def _linear(N, K, seed, pmin=33):
    mq = _mq()
    wb = workloads.random_bf16((N, K), seed, 0.02)
    lin = mq.Linear(to_dev_bf16(wb), prefill_min_rows=pmin).prepare()
    return lin, wb


def _same(a, b):
    import torch
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("N,K", [(300, 512), (1024, 4096)])
def test_prepare_is_the_oracle_quantization(N, K):
    announce("linear prepare", N, K)
    import torch
    lin, wb = _linear(N, K, 7 + N)
    torch.cuda.synchronize()
    codes, scales, st = quantized_host(lin.w_nvfp4)
    ref = oracle.quantize_nvfp4(wb)
    assert st == int(np.float32(ref.s_t).view(np.uint32))
    assert np.array_equal(scales, ref.scales)
    assert np.array_equal(codes, ref.codes)


@pytest.mark.parametrize("M", [1, 7, 16, 32])
def test_decode_calls_take_the_bf16_gemv(M):
    announce("linear decode", M)
    import torch
    mq = _mq()
    N, K = 1024, 4096
    lin, wb = _linear(N, K, 11)
    xb = workloads.random_bf16((M, K), 12 + M)
    x = to_dev_bf16(xb)
    assert lin.path(M) == mq.MQ_PATH_DECODE_BF16
    y = lin.forward(x)
    y_direct = mq.decode_linear(x, lin.w_bf16)
    torch.cuda.synchronize()
    assert _same(y, y_direct)
    ref = oracle.gemv_bf16_ref(workloads.bf16_bits_to_f32(xb), workloads.bf16_bits_to_f32(wb))
    r = rule_t(bf16_dev_to_f64(y), ref, bf16_out=True)
    print("  rule T:", r, flush=True)
    assert r.ok, str(r)


@pytest.mark.parametrize("M,fused", [(33, False), (33, True), (256, False), (300, True)])
def test_prefill_calls_take_the_nvfp4_gemm(M, fused):
    announce("linear prefill", M, fused)
    import torch
    mq = _mq()
    N, K = 1024, 4096
    lin, wb = _linear(N, K, 21)
    xb = workloads.random_bf16((M, K), 22 + M, 1.0, "lognormal_mixed")
    x = to_dev_bf16(xb)
    assert lin.path(M) == mq.MQ_PATH_PREFILL_NVFP4
    flags = mq.MQ_A_FUSED_BF16 if fused else 0
    y = lin.forward(x, flags=flags)
    y_direct = mq.prefill_linear(x, lin.w_nvfp4, fused=fused)
    torch.cuda.synchronize()
    assert _same(y, y_direct)
    ref = oracle.gemm_nvfp4_ref(oracle.quantize_nvfp4(xb), oracle.quantize_nvfp4(wb))
    r = rule_t(bf16_dev_to_f64(y), ref, bf16_out=True)
    print("  rule T:", r, flush=True)
    assert r.ok, str(r)


def test_phase_flags_override_the_row_count():
    # a one-token prefill goes through NVFP4; with prefill_min_rows = 1 a
    # decode step still takes BF16 when it says so
    announce("linear phase flags")
    import torch
    mq = _mq()
    N, K = 512, 1024
    lin, wb = _linear(N, K, 31, pmin=1)
    xb = workloads.random_bf16((5, K), 32)
    x = to_dev_bf16(xb)
    assert lin.path(5) == mq.MQ_PATH_PREFILL_NVFP4
    assert lin.path(5, mq.MQ_PHASE_DECODE) == mq.MQ_PATH_DECODE_BF16
    y_dec = lin.forward(x, flags=mq.MQ_PHASE_DECODE)
    y_pre = lin.forward(x)
    assert _same(y_dec, mq.decode_linear(x, lin.w_bf16))
    assert _same(y_pre, mq.prefill_linear(x, lin.w_nvfp4))
    lin.prefill_min_rows = 33
    x1 = x[:1].contiguous()
    y1 = lin.forward(x1, flags=mq.MQ_PHASE_PREFILL)
    torch.cuda.synchronize()
    assert _same(y1, mq.prefill_linear(x1, lin.w_nvfp4))
    x40 = to_dev_bf16(workloads.random_bf16((40, K), 33))
    with pytest.raises(mq.MQError):
        lin.forward(x40, flags=mq.MQ_PHASE_DECODE)


def test_decode_and_prefill_outputs_differ_as_the_formats_do():
    # the two paths compute the same linear in different precisions: the
    # BF16 path is within rule T of the exact bf16 product, the NVFP4 path of
    # the exact product of the quantized operands; against the unquantized
    # product the NVFP4 path's error is the quantization error
    announce("linear precision split")
    mq = _mq()
    N, K = 512, 2048
    lin, wb = _linear(N, K, 41)
    xb = workloads.random_bf16((16, K), 42)
    x = to_dev_bf16(xb)
    exact = oracle.gemv_bf16_ref(workloads.bf16_bits_to_f32(xb), workloads.bf16_bits_to_f32(wb))
    y_dec = bf16_dev_to_f64(lin.forward(x, flags=mq.MQ_PHASE_DECODE))
    y_pre = bf16_dev_to_f64(lin.forward(x, flags=mq.MQ_PHASE_PREFILL))
    rel = lambda y: float(np.linalg.norm(y - exact) / np.linalg.norm(exact))
    print(f"  rel_fro decode {rel(y_dec):.2e} prefill {rel(y_pre):.2e}", flush=True)
    assert rel(y_dec) < 4e-3
    assert rel(y_pre) > 5 * rel(y_dec)
