"""GPU checks of mq_gemm_nvfp4_prefill_fused_noalloc, the allocation-free
variant of the fused-prologue GEMM (the activation's scale record and NVFP4
copy live in the library's own scratch buffer).

Its output must equal, bit for bit, what the existing entry point
mq_gemm_nvfp4_prefill with MQ_A_FUSED_BF16 writes with caller-owned buffers
(the same kernels run), over two calls in a row on the shared buffer, the
second smaller than the first, in both forms the fused path takes (the
quantize-once panel form, forced at these sizes through a test knob, and the
encode pass then the plain GEMM, the default here and for ragged K) and
both output types; one case is also held to the oracle.
"""

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import announce, bf16_dev_to_f64, to_dev_bf16
from tests.parity import rule_t

pytestmark = pytest.mark.gpu


def _mq():
    import fp4_block_scaled_elem_amd as mq
    return mq


def _case(M, N, K, seed, f32=False):
    import torch
    mq = _mq()
    xa = workloads.random_bf16((M, K), seed, 1.0, "lognormal_mixed")
    xw = workloads.random_bf16((N, K), seed + 1, 0.02)
    x = to_dev_bf16(xa)
    w = mq.quantize(to_dev_bf16(xw))
    dt = torch.float32 if f32 else torch.bfloat16
    flags = mq.MQ_OUT_F32 if f32 else 0
    c_na = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
    mq.mq_gemm_nvfp4_prefill_fused_noalloc(x, w, c_na, flags)
    c_ref = torch.empty((M, N), dtype=dt, device="cuda")
    mq.mq_gemm_nvfp4_prefill(mq.NVFP4.empty(M, K), x, w, c_ref, flags | mq.MQ_A_FUSED_BF16)
    torch.cuda.synchronize()
    v = torch.int32 if f32 else torch.int16
    assert torch.equal(c_na.view(v), c_ref.view(v)), f"{M}x{N}x{K}: output differs from the existing entry point"
    return xa, xw, c_na


@pytest.mark.parametrize("f32", [False, True], ids=["bf16", "f32"])
def test_two_calls_second_smaller(f32):
    announce("noalloc two calls", "f32" if f32 else "bf16")
    mq = _mq()
    # at these sizes the library takes the encode pass and the plain GEMM by
    # default; the threshold knob forces the panel form for the first two
    old = mq.mq_check_set_panel_min_tiles(1)
    try:
        xa, xw, c = _case(1000, 520, 1024, 11, f32)  # quantize-once panel form, 4 panels
        _case(300, 300, 512, 12, f32)                 # smaller, same form
    finally:
        mq.mq_check_set_panel_min_tiles(old)
    _case(1000, 520, 1024, 14, f32)                   # default: encode pass, then the plain GEMM
    _case(130, 200, 272, 13, f32)                     # ragged K: encode pass, then the plain GEMM
    if not f32:
        r = rule_t(bf16_dev_to_f64(c), oracle.gemm_nvfp4_ref(oracle.quantize_nvfp4(xa), oracle.quantize_nvfp4(xw)),
                   bf16_out=True)
        print("  rule T:", r, flush=True)
        assert r.ok, str(r)


def test_largest_size_then_small():
    announce("noalloc at the size limit, then small")
    mq = _mq()
    M, K = mq.MQ_NOALLOC_MAX_ELEMS // 4096, 4096    # exactly the scratch capacity
    _case(M, 256, K, 21)
    _case(64, 128, 256, 22)


def test_rejects_too_large():
    announce("noalloc rejects sizes past its scratch")
    import torch
    mq = _mq()
    M, K = mq.MQ_NOALLOC_MAX_ELEMS // 4096 + 1, 4096
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    w = mq.quantize(torch.zeros((16, K), dtype=torch.bfloat16, device="cuda"))
    c = torch.empty((M, 16), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mq.MQError) as e:
        mq.mq_gemm_nvfp4_prefill_fused_noalloc(x, w, c)
    assert e.value.status == mq.MQ_ERR_SHAPE
