"""GPU parity beyond 2^31 elements: index arithmetic at the largest sizes.

Each case builds a tensor of more than 2^31 elements on the device from a
small bank of seeded rows (row r is bank row r mod P, P prime and not a
divisor of any tile size), so the oracle only has to process the bank: every
output row of a row-wise operation equals the oracle's output for its bank
row.  Element offsets past 2^31 (and byte offsets past 2^32 for bf16) are
where a 32-bit index would wrap, so the rows there are always among those
compared.

* Quantizer: the whole code and scale output is compared bit for bit with
  the oracle's, expanded by the same row map; the tensor's largest magnitude
  is planted in the last row, past 2^31 elements, so the amax pass has to
  reach it for s_t to match.
* GEMM (C of more than 2^31 elements, with uploaded operands for the
  whole-stage and the ragged-K kernels, and the fused quantize-once form):
  rule T on every column of sampled rows, including all rows whose output
  offsets lie past 2^31; the fused form's NVFP4 copy of A is compared whole,
  bit for bit.
* Decode GEMV (W of more than 2^31 elements): rule T on the whole output.
"""

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import announce, bf16_dev_to_f64, to_dev_bf16
from tests.parity import rule_t

pytestmark = pytest.mark.gpu

TWO31 = 1 << 31


def _mq():
    import fp4_block_scaled_elem_amd as mq
    return mq


def _fresh():
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _row_map(rows, period):
    import torch
    return torch.arange(rows, device="cuda") % period


def _expand(bank_np, idx):
    """Device tensor whose row r is bank_np[idx[r]]."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(bank_np)).cuda().index_select(0, idx)


def test_quantize_beyond_2_31_elements():
    import torch
    mq = _mq()
    _fresh()
    R, K, P = 131075, 16400, 251
    assert R * K > TWO31
    bank = workloads.random_bf16((P, K), 31, 1.0, "lognormal_mixed")
    planted = bank[0].copy()
    big = workloads.bf16_bits_to_f32(bank).astype(np.float64)
    peak = np.float32(2.0 * np.abs(big).max())        # a power-of-two multiple: exact in bf16
    planted[K - 1] = workloads.f32_to_bf16_bits(np.array([peak], np.float32))[0]
    small = np.vstack([bank, planted[None, :]])
    ref = oracle.quantize_nvfp4(small)                # same rows, same maximum as the big tensor
    announce("large quantize", R, K, "elements", R * K)
    idx = _row_map(R, P)
    idx[R - 1] = P                                    # the planted row
    x = _expand(small.view(np.int16), idx).view(torch.bfloat16)
    q = mq.NVFP4.empty(R, K)
    mq.mq_quantize_nvfp4(x, q)
    torch.cuda.synchronize()
    del x
    got_st = int(q.rec[:1].cpu().numpy().view(np.uint32)[0])
    assert got_st == int(np.float32(ref.s_t).view(np.uint32)), "tensor scale differs"
    codes_ok = torch.equal(q.codes, _expand(ref.codes, idx))
    scales_ok = torch.equal(q.scales, _expand(ref.scales, idx))
    assert codes_ok and scales_ok, (codes_ok, scales_ok)
    # the last rows, spelled out (past 2^31 elements)
    last = q.codes[R - 2:].cpu().numpy()
    assert np.array_equal(last[0], ref.codes[(R - 2) % P]) and np.array_equal(last[1], ref.codes[P])
    del q
    _fresh()


def _gemm_case(M, N, K, fused):
    import torch
    mq = _mq()
    PA, PW = 251, 241
    xa = workloads.random_bf16((PA, K), 41 + K, 1.0, "normal")
    xw = workloads.random_bf16((PW, K), 43 + K, 0.02, "normal")
    oa, ow = oracle.quantize_nvfp4(xa), oracle.quantize_nvfp4(xw)
    cbank = oracle.gemm_nvfp4_ref(oa, ow)             # [PA][PW] float64
    idx_m, idx_n = _row_map(M, PA), _row_map(N, PW)
    w = mq.NVFP4(_expand(ow.codes, idx_n), _expand(ow.scales, idx_n),
                 torch.zeros(mq.REC_BYTES // 4, dtype=torch.int32, device="cuda"))
    w.set_s_t(float(ow.s_t))
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    announce("large gemm", M, N, K, "fused" if fused else "uploaded", "outputs", M * N)
    if fused:
        x = _expand(xa.view(np.int16), idx_m).view(torch.bfloat16)
        keep = mq.NVFP4.empty(M, K)
        mq.mq_gemm_nvfp4_prefill(keep, x, w, c, mq.MQ_A_FUSED_BF16)
        torch.cuda.synchronize()
        del x
        assert int(keep.rec[:1].cpu().numpy().view(np.uint32)[0]) == int(np.float32(oa.s_t).view(np.uint32))
        assert torch.equal(keep.codes, _expand(oa.codes, idx_m)), "A's codes differ"
        assert torch.equal(keep.scales, _expand(oa.scales, idx_m)), "A's scales differ"
        del keep
    else:
        a = mq.NVFP4(_expand(oa.codes, idx_m), _expand(oa.scales, idx_m),
                     torch.zeros(mq.REC_BYTES // 4, dtype=torch.int32, device="cuda"))
        a.set_s_t(float(oa.s_t))
        mq.mq_gemm_nvfp4_prefill(a, None, w, c, 0)
        torch.cuda.synchronize()
        del a
    first_past = (TWO31 + N - 1) // N                 # first row with an output offset past 2^31
    rng = np.random.default_rng([M, N, K])
    rows = np.unique(np.concatenate([np.arange(4), rng.choice(M, 200, replace=False),
                                     np.arange(min(first_past, M - 130), M)]))
    assert rows[-1] == M - 1 and np.any(rows * N >= TWO31)
    got = bf16_dev_to_f64(c.index_select(0, torch.from_numpy(rows).cuda()))
    del c
    cols = np.arange(N) % PW
    ref = cbank[rows % PA][:, cols]
    r = rule_t(got, ref, bf16_out=True)
    print("  rule T:", r, flush=True)
    assert r.ok, str(r)
    _fresh()


@pytest.mark.parametrize("K", [256, 144])
def test_gemm_output_beyond_2_31_elements(K):
    _fresh()
    M, N = 65600, 32800
    assert M * N > TWO31
    _gemm_case(M, N, K, fused=False)


def test_gemm_fused_quantize_once_beyond_2_31_elements():
    _fresh()
    M, N, K = 65600, 32800, 256
    _gemm_case(M, N, K, fused=True)


@pytest.mark.parametrize("M", [3, 32])
def test_gemv_weight_beyond_2_31_elements(M):
    import torch
    mq = _mq()
    _fresh()
    N, K, P = 262160, 8192, 241
    assert N * K > TWO31
    wb = workloads.random_bf16((P, K), 47, 0.02, "normal")
    xb = workloads.random_bf16((M, K), 53 + M, 1.0, "normal")
    ybank = oracle.gemv_bf16_ref(workloads.bf16_bits_to_f32(xb), workloads.bf16_bits_to_f32(wb))
    announce("large gemv", M, N, K, "weights", N * K)
    idx = _row_map(N, P)
    w = _expand(wb.view(np.int16), idx).view(torch.bfloat16)
    x = to_dev_bf16(xb)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mq.mq_gemv_bf16_decode(x, w, y)
    torch.cuda.synchronize()
    del w
    got = bf16_dev_to_f64(y)
    ref = ybank[:, np.arange(N) % P]
    r = rule_t(got, ref, bf16_out=True)
    print("  rule T:", r, flush=True)
    assert r.ok, str(r)
    _fresh()
