"""HIP-graph capture of the library's calls (torch.cuda.CUDAGraph around the
C-ABI entry points).

The entry points only queue kernel launches on the caller's stream: no
allocation, no memset, no host synchronisation, so a serving loop can
capture a prefill or decode step once and replay it.  Each graph here is
replayed several times; before every replay its inputs are overwritten
eagerly with new data, and after it the outputs must equal, bit for bit,
eager calls of the library on the same data (which also put eager work of
the library between the replays).
"""

import pytest

import workloads
from tests.gpu_util import announce, to_dev_bf16

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _mq():
    import fp4_block_scaled_elem_amd as mq
    return mq


def _capture(fn):
    """fn() once eagerly on a side stream (first calls set per-kernel
    attributes), then captured into a graph."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def _same(a, b):
    import torch
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    return torch.equal(a, b)


def test_prefill_quantize_and_gemm_replay():
    announce("graph: quantize + gemm")
    import torch
    mq = _mq()
    M, K, N = 300, 1024, 520
    w = mq.quantize(to_dev_bf16(workloads.random_bf16((N, K), 1, 0.02)))
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    x.copy_(to_dev_bf16(workloads.random_bf16((M, K), 2, 1.0, "lognormal_mixed")))
    qa = mq.NVFP4.empty(M, K)
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step():
        mq.mq_quantize_nvfp4(x, qa)
        mq.mq_gemm_nvfp4_prefill(qa, None, w, c)

    g = _capture(step)
    for r in range(REPLAYS):
        xr = to_dev_bf16(workloads.random_bf16((M, K), 10 + r, 1.0 + r, "lognormal_mixed"))
        x.copy_(xr)
        g.replay()
        qe = mq.quantize(xr)
        ce = torch.empty_like(c)
        mq.mq_gemm_nvfp4_prefill(qe, None, w, ce)
        torch.cuda.synchronize()
        assert _same(qa.codes, qe.codes) and _same(qa.scales, qe.scales), f"replay {r}: quantization"
        assert _same(qa.rec[:1], qe.rec[:1]), f"replay {r}: tensor scale"
        assert _same(c, ce), f"replay {r}: gemm output"


def test_single_launch_quantizer_replay():
    # The single-launch quantizer (inputs of 17 to 64 half-groups per lane,
    # here 4096 x 5120 on 256 CUs) takes its barrier epoch from the record on
    # the device, so every replay of a captured call is a new epoch.  Each
    # replay's input has a smaller maximum than the last (a slot left from an
    # earlier epoch would raise the scale), and an eager call on the same
    # record runs between replays.
    announce("graph: single-launch quantizer")
    import torch
    mq = _mq()
    M, K = 4096, 5120
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    x.copy_(to_dev_bf16(workloads.random_bf16((M, K), 40, 64.0)))
    qa = mq.NVFP4.empty(M, K)
    g = _capture(lambda: mq.mq_quantize_nvfp4(x, qa))
    for r in range(REPLAYS):
        xr = to_dev_bf16(workloads.random_bf16((M, K), 41 + r, 32.0 / 4 ** r))
        x.copy_(xr)
        g.replay()
        qe = mq.quantize(xr)
        torch.cuda.synchronize()
        assert _same(qa.codes, qe.codes) and _same(qa.scales, qe.scales), f"replay {r}: quantization"
        assert _same(qa.rec[:1], qe.rec[:1]), f"replay {r}: tensor scale"
        # an eager call on the captured record between replays
        mq.mq_quantize_nvfp4(to_dev_bf16(workloads.random_bf16((M, K), 60 + r, 100.0)), qa)
    torch.cuda.synchronize()
    assert mq.mq_check_quant_gave_up() == 0


@pytest.mark.parametrize("form", ["tile", "panel"])
def test_fused_prologue_gemm_replay(form):
    # tile: A re-quantized per column tile; panel: quantized once per
    # workgroup into A's NVFP4 buffers (the quantize-once kernel)
    announce("graph: fused-prologue gemm", form)
    import torch
    mq = _mq()
    M, K, N = 256, 512, 512
    w = mq.quantize(to_dev_bf16(workloads.random_bf16((N, K), 3, 0.02)))
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    x.copy_(to_dev_bf16(workloads.random_bf16((M, K), 4, 1.0)))
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    rec = torch.zeros(mq.REC_BYTES // 4, dtype=torch.int32, device="cuda")
    keep = mq.NVFP4.empty(M, K) if form == "panel" else None
    # one panel of two column tiles: the panel form only when forced (by
    # default this shape takes the encode pass and the plain GEMM)
    old = mq.mq_check_set_panel_min_tiles(1)
    try:
        g = _capture(lambda: mq.prefill_linear(x, w, out=c, fused=True, rec=rec, keep_a=keep))
    finally:
        mq.mq_check_set_panel_min_tiles(old)
    for r in range(REPLAYS):
        xr = to_dev_bf16(workloads.random_bf16((M, K), 20 + r, 0.5 + r, "lognormal_mixed"))
        x.copy_(xr)
        g.replay()
        ce = mq.prefill_linear(xr, w)           # two-pass quantizer + plain GEMM: the same bits
        torch.cuda.synchronize()
        assert _same(c, ce), f"replay {r}"


def test_decode_gemvs_replay():
    announce("graph: bf16 and nvfp4 decode gemv")
    import torch
    mq = _mq()
    M, K, N = 5, 1024, 700
    wb = to_dev_bf16(workloads.random_bf16((N, K), 5, 0.02))
    wq = mq.quantize(wb)
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    x.copy_(to_dev_bf16(workloads.random_bf16((M, K), 6, 1.0)))
    xq = mq.NVFP4.empty(M, K)
    y1 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step():
        mq.mq_gemv_bf16_decode(x, wb, y1)
        mq.mq_quantize_nvfp4(x, xq)
        mq.mq_gemv_nvfp4_decode(xq, wq, y2)

    g = _capture(step)
    for r in range(REPLAYS):
        xr = to_dev_bf16(workloads.random_bf16((M, K), 30 + r, 1.0))
        x.copy_(xr)
        g.replay()
        e1 = mq.decode_linear(xr, wb)
        e2 = torch.empty_like(y2)
        mq.mq_gemv_nvfp4_decode(mq.quantize(xr), wq, e2)
        torch.cuda.synchronize()
        assert _same(y1, e1), f"replay {r}: bf16 gemv"
        assert _same(y2, e2), f"replay {r}: nvfp4 gemv"


@pytest.mark.parametrize("M", [4, 64])
def test_phase_aware_linear_replay(M):
    # M = 4 takes the BF16 decode path, M = 64 the NVFP4 prefill path
    announce("graph: phase-aware linear", M)
    import torch
    mq = _mq()
    K, N = 1024, 384
    lin = mq.Linear(to_dev_bf16(workloads.random_bf16((N, K), 7, 0.02))).prepare()
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    x.copy_(to_dev_bf16(workloads.random_bf16((M, K), 8, 1.0)))
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    a_work = mq.NVFP4.empty(M, K)
    g = _capture(lambda: lin.forward(x, out=y, a_work=a_work))
    for r in range(REPLAYS):
        xr = to_dev_bf16(workloads.random_bf16((M, K), 40 + r, 1.0, "lognormal_mixed"))
        x.copy_(xr)
        g.replay()
        ye = lin.forward(xr)
        torch.cuda.synchronize()
        assert _same(y, ye), f"replay {r}"


def test_rmsnorm_quantize_replay():
    # the RMSNorm fused with quantization: both passes captured; each replay
    # on new data equals the eager call bit for bit
    announce("graph: rmsnorm fused with quantization")
    import torch
    mq = _mq()
    M, K = 256, 4096
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    x.copy_(to_dev_bf16(workloads.random_bf16((M, K), 50, 1.0, "lognormal_mixed")))
    g = to_dev_bf16(workloads.random_bf16((K,), 51, 1.0))
    q = mq.NVFP4.empty(M, K)
    graph = _capture(lambda: mq.mq_rmsnorm_quantize_nvfp4(x, g, q))
    for r in range(REPLAYS):
        xr = to_dev_bf16(workloads.random_bf16((M, K), 52 + r, 4.0 ** r, "lognormal_mixed"))
        x.copy_(xr)
        graph.replay()
        qe = mq.NVFP4.empty(M, K)
        mq.mq_rmsnorm_quantize_nvfp4(xr, g, qe)
        torch.cuda.synchronize()
        assert torch.equal(q.codes, qe.codes) and torch.equal(q.scales, qe.scales), f"replay {r}"
        assert torch.equal(q.rec[:1], qe.rec[:1]), f"replay {r}: s_t"
