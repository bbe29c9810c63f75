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
    # M > 16 with at least 256 workgroups of 32 W rows: the two-row-tile
    # workgroups, the last one's second tile partly or wholly past N
    (32, 8200, 256), (20, 8197, 384), (17, 8208, 128),
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


@pytest.mark.parametrize("M,Ns,K", [
    (1, (4096, 1024, 1024), 4096),         # a decode step's q, k and v as one launch
    (32, (14336, 14336), 4096),           # gate and up
    (5, (17, 300, 1, 48), 512),           # ragged row counts, four groups
    (17, (1000, 33), 4112),               # K % 128 != 0: the register-path kernel
    # 32 W rows per workgroup in the grouped launch, 16 in the single calls
    (32, (5000, 3300), 4096), (17, (8200, 48), 1024),
    # on 256 CUs: 64 W rows on four waves in the grouped launch, 32 and 16
    # rows on eight waves in the single calls
    (24, (8192, 4096), 1024),
])
def test_grouped_bit_identical_to_single_calls(M, Ns, K):
    # one launch over several weights that read the same X: every output is
    # the single call's, bit for bit (and the single calls are held to the
    # oracle above); the first group is also checked against the oracle
    announce("gemv grouped", M, Ns, K)
    import torch
    import fp4_block_scaled_elem_amd as mq
    xb = workloads.random_bf16((M, K), 300 + M, 1.0)
    wbs = [workloads.random_bf16((n, K), 400 + i, 0.02) for i, n in enumerate(Ns)]
    x = to_dev_bf16(xb)
    ws = [to_dev_bf16(wb) for wb in wbs]
    ys = [torch.empty((M, n), dtype=torch.bfloat16, device="cuda") for n in Ns]
    mq.mq_gemv_bf16_decode_grouped(x, ws, ys)
    singles = [mq.decode_linear(x, w) for w in ws]
    torch.cuda.synchronize()
    for g, (y, y1) in enumerate(zip(ys, singles)):
        assert torch.equal(y.view(torch.int16), y1.view(torch.int16)), f"group {g}"
    ref = oracle.gemv_bf16_ref(workloads.bf16_bits_to_f32(xb), workloads.bf16_bits_to_f32(wbs[0]))
    r = rule_t(bf16_dev_to_f64(ys[0]), ref, bf16_out=True)
    assert r.ok, str(r)


@pytest.mark.parametrize("M,N_big,N_small,K", [
    (3, 4096, 4080, 1024),    # 256 vs 255 workgroups: non-temporal W copies on one side only
    (32, 8192, 8160, 512),    # 256 vs 255 pairs of row tiles: 32-row vs 16-row workgroups
    (20, 8192, 8160, 384),
    # on 256 CUs: 192 vs 191 tiles of 64 rows: four-wave 64-row workgroups
    # (each wave standing for two of the eight-wave form) vs 32-row ones
    (32, 12288, 12224, 1024),
    (17, 12288, 12224, 4096),
])
def test_dispatch_boundaries_agree(M, N_big, N_small, K):
    # the launch choices at these boundaries change cache policy or rows per
    # workgroup, not arithmetic: the rows both weights share give the same bits
    announce("gemv boundary", M, N_big, N_small, K)
    import torch
    import fp4_block_scaled_elem_amd as mq
    xb = workloads.random_bf16((M, K), 700 + M, 1.0)
    wb = workloads.random_bf16((N_big, K), 701 + K, 0.02)
    x, w = to_dev_bf16(xb), to_dev_bf16(wb)
    y_big = mq.decode_linear(x, w)
    y_small = mq.decode_linear(x, w[:N_small].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(y_big[:, :N_small].contiguous().view(torch.int16), y_small.view(torch.int16))
    ref = oracle.gemv_bf16_ref(workloads.bf16_bits_to_f32(xb), workloads.bf16_bits_to_f32(wb))
    r = rule_t(bf16_dev_to_f64(y_big), ref, bf16_out=True)
    assert r.ok, str(r)
