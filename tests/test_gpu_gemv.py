"""GPU parity of mq_gemv_bf16_decode against the float64 oracle."""

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import announce, bf16_dev_to_f64, to_dev_bf16
from tests.parity import rule_t

pytestmark = pytest.mark.gpu


def _gemv(xb, wb):
    import torch
    import fp4_block_scaled_elem_amd as mq
    x, w = to_dev_bf16(xb), to_dev_bf16(wb)
    y = torch.empty((xb.shape[0], wb.shape[0]), dtype=torch.bfloat16, device="cuda")
    mq.mq_gemv_bf16_decode(x, w, y)
    torch.cuda.synchronize()
    return bf16_dev_to_f64(y)


def _check(xb, wb):
    ref = oracle.gemv_bf16_ref(workloads.bf16_bits_to_f32(xb), workloads.bf16_bits_to_f32(wb))
    r = rule_t(_gemv(xb, wb), ref, bf16_out=True)
    print("  rule T:", r, flush=True)
    assert r.ok, str(r)


@pytest.mark.parametrize("M", [1, 4, 16, 32])
@pytest.mark.parametrize("proj", ["q", "k", "gate", "down"])
def test_cfg4_decode(M, proj):
    announce("gemv cfg4", M, proj)
    act = workloads.PROJ_INPUT[proj]
    _check(workloads.activation(4, act, M=M), workloads.weight(4, proj))


@pytest.mark.parametrize("M,N,K", [
    # K % 128 != 0: the register-path kernel
    (1, 1, 16), (3, 17, 48), (17, 1000, 4112), (32, 33, 160), (5, 4096, 16),
    # K % 128 == 0: the LDS-ring kernel, with ragged N and M, one chunk (three
    # waves without work), and chunk counts that do not divide by four
    (31, 64, 8192), (1, 1, 128), (17, 1000, 1024), (32, 4100, 256), (2, 33, 384), (16, 17, 640),
])
def test_ragged(M, N, K):
    announce("gemv ragged", M, N, K)
    _check(workloads.random_bf16((M, K), M + N, 1.0), workloads.random_bf16((N, K), K, 0.02))


@pytest.mark.parametrize("M", list(range(1, 33)))
def test_every_row_count(M):
    # every M in 1..32: the ring kernel copies only the X row groups below M
    # (one copy per four rows) and takes 32 W rows per workgroup above 16;
    # N = 48 and 17 leave the last workgroup's second W tile partly or
    # almost entirely past N
    N = 48 if M % 2 else 17
    announce("gemv rows", M, N)
    _check(workloads.random_bf16((M, 512), 100 + M, 1.0), workloads.random_bf16((N, 512), 200 + M, 0.02))


def test_one_hot_rows_are_exact():
    announce("gemv one-hot")
    M, N, K = 20, 300, 1024
    cols = [0, 1, 15, 16, 127, 128, 511, 1023, 300, 77, 5, 900, 640, 641, 1000, 999, 3, 256, 257, 768]
    x = np.zeros((M, K), np.float32)
    for m, k in enumerate(cols):
        x[m, k] = 1.0
    wb = workloads.random_bf16((N, K), 3)
    y = _gemv(workloads.f32_to_bf16_bits(x), wb)
    w = workloads.bf16_bits_to_f32(wb).astype(np.float64)
    for m, k in enumerate(cols):
        assert np.array_equal(y[m], w[:, k]), m


def test_deterministic():
    announce("gemv determinism")
    xb, wb = workloads.random_bf16((32, 4096), 1), workloads.random_bf16((1024, 4096), 2, 0.02)
    assert np.array_equal(_gemv(xb, wb), _gemv(xb, wb))
