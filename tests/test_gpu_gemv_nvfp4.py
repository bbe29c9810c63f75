"""GPU parity of mq_gemv_nvfp4_decode (X and W both NVFP4, M <= 32) against
the float64 oracle: the exact product of the dequantized operands, compared
element by element under rule T.  Operands come from the oracle's
quantization (uploaded), so the test covers the kernel alone."""

import functools

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import announce, bf16_dev_to_f64, upload_nvfp4
from tests.parity import rule_t

pytestmark = pytest.mark.gpu


def _gemv(oa, ow):
    import torch
    import fp4_block_scaled_elem_amd as mq
    M, N = oa.shape[0], ow.shape[0]
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mq.mq_gemv_nvfp4_decode(upload_nvfp4(oa), upload_nvfp4(ow), y)
    torch.cuda.synchronize()
    return bf16_dev_to_f64(y)


def _check(xb, wb=None, ow=None):
    oa = oracle.quantize_nvfp4(xb)
    ow = ow if ow is not None else oracle.quantize_nvfp4(wb)
    r = rule_t(_gemv(oa, ow), oracle.gemm_nvfp4_ref(oa, ow), bf16_out=True)
    print("  rule T:", r, flush=True)
    assert r.ok, str(r)


@functools.lru_cache(maxsize=None)
def _cfg4_weight(proj):
    return oracle.quantize_nvfp4(workloads.weight(4, proj))


@pytest.mark.parametrize("M", [1, 16, 32])
@pytest.mark.parametrize("proj", ["q", "k", "gate", "down"])
def test_cfg4_decode(M, proj):
    announce("gemv nvfp4 cfg4", M, proj)
    _check(workloads.activation(4, workloads.PROJ_INPUT[proj], M=M), ow=_cfg4_weight(proj))


@pytest.mark.parametrize("M,N,K", [
    # K % 256 == 0: whole-chunk loads; ragged N and M, fewer chunks than waves
    (1, 1, 256), (3, 17, 512), (17, 100, 2048), (32, 33, 768), (31, 4100, 256),
    # other K: group-by-group loads, each bounds-checked
    (1, 1, 16), (5, 100, 272), (32, 33, 4112), (17, 1000, 1040), (2, 64, 48),
])
def test_ragged(M, N, K):
    announce("gemv nvfp4 ragged", M, N, K)
    _check(workloads.random_bf16((M, K), M + N + K, 1.0, "lognormal_mixed"), workloads.random_bf16((N, K), K, 0.02))


def test_identity_weight_picks_rows_exactly():
    # W = 2688 I quantizes exactly (s_t = 1, every group scale 448, value 6),
    # so each output element is one product of dequantized values, exact in
    # binary32 (X's tensor scale is a power of two); the bf16 output must be
    # the nearest-even bf16 of the oracle's exact value
    announce("gemv nvfp4 identity")
    K = 512
    w = workloads.f32_to_bf16_bits(np.eye(K, dtype=np.float32) * np.float32(2688.0))
    rng = np.random.default_rng(5)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float32)
    x = grid[rng.integers(0, 8, (9, K))] * np.where(rng.random((9, K)) < 0.5, -1, 1).astype(np.float32)
    x[:, 0] = 6.0 * 448.0 / 64.0
    xb = workloads.f32_to_bf16_bits(x.astype(np.float32))
    oa, ow = oracle.quantize_nvfp4(xb), oracle.quantize_nvfp4(w)
    ref = oracle.gemm_nvfp4_ref(oa, ow)
    assert np.array_equal(ref, ref.astype(np.float32).astype(np.float64))
    want = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(ref.astype(np.float32))).astype(np.float64)
    assert np.array_equal(_gemv(oa, ow), want)


def test_deterministic():
    announce("gemv nvfp4 determinism")
    oa = oracle.quantize_nvfp4(workloads.random_bf16((32, 4096), 1))
    ow = oracle.quantize_nvfp4(workloads.random_bf16((1024, 4096), 2, 0.02))
    assert np.array_equal(_gemv(oa, ow), _gemv(oa, ow))
