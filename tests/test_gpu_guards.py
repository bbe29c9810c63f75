"""Guard bytes around every output, on a non-default stream.

Each output buffer (codes, scale bytes, scale records, bf16 / binary32
results) sits inside a larger allocation whose 256 bytes before and after it
are filled with 0xA5; every entry point runs on ragged shapes (rows and
columns that leave partial tiles, workgroups and chunks) on a stream of its
own, after which the guards must be intact.  Floating-point outputs are
pre-filled with NaN, so an element left unwritten shows as well; the codes
and scale bytes written by the fused GEMM's quantize-once form must equal the
standalone quantizer's.
"""

import numpy as np
import pytest

import workloads
from tests.gpu_util import announce, to_dev_bf16

pytestmark = pytest.mark.gpu

G = 256           # guard bytes on each side
PAT = 0xA5


class Guarded:
    """A view of `shape` and `dtype` inside a guarded byte buffer (`tail`
    guard bytes after it, G before)."""

    def __init__(self, shape, dtype, fill=None, tail=G):
        import torch
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.n = n
        self.buf = torch.full((G + n + tail,), PAT, dtype=torch.uint8, device="cuda")
        self.t = self.buf[G:G + n].view(dtype).view(*shape)
        if fill is not None:
            self.t.view(torch.uint8).fill_(fill)

    def intact(self):
        import torch
        head, tail = self.buf[:G], self.buf[G + self.n:]
        return bool(torch.all(head == PAT)) and bool(torch.all(tail == PAT))

    def written(self):
        import torch
        return not bool(torch.isnan(self.t.float()).any())


def _nvfp4(rows, cols):
    import torch
    import fp4_block_scaled_elem_amd as mq
    c = Guarded((rows, cols // 2), torch.uint8)
    s = Guarded((rows, cols // 16), torch.uint8)
    r = Guarded((mq.REC_BYTES // 4,), torch.int32, fill=0)
    return mq.NVFP4(c.t, s.t, r.t), (c, s, r)


def _all_intact(gs):
    return all(g.intact() for g in gs)


@pytest.mark.parametrize("rows,cols", [(2999, 7184), (4000, 14336)])
def test_single_launch_quantizer_stays_inside_its_buffers(rows, cols):
    # ragged shares of 21 (32 kept in registers) and 55 (48 in registers, the
    # rest held in LDS) half-groups per lane on 256 CUs: the lanes past the
    # input in the last share compute codes that must be dropped, not
    # written up to hundreds of KB past the buffers, hence the 1 MB tail guards
    announce("guards single-launch quantizer", rows, cols)
    import torch
    import fp4_block_scaled_elem_amd as mq
    x = to_dev_bf16(workloads.random_bf16((rows, cols), 90, 1.0, "lognormal_mixed"))
    c = Guarded((rows, cols // 2), torch.uint8, tail=1 << 20)
    sc = Guarded((rows, cols // 16), torch.uint8, tail=1 << 20)
    r = Guarded((mq.REC_BYTES // 4,), torch.int32, fill=0)
    q = mq.NVFP4(c.t, sc.t, r.t)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        mq.mq_quantize_nvfp4(x, q)
    st.synchronize()
    assert _all_intact([c, sc, r])
    ref = mq.quantize(x)
    torch.cuda.synchronize()
    assert torch.equal(c.t, ref.codes) and torch.equal(sc.t, ref.scales)


@pytest.mark.parametrize("M,N,K", [(37, 300, 272), (300, 520, 512), (129, 17, 4112)])
def test_prefill_paths_stay_inside_their_buffers(M, N, K):
    announce("guards prefill", M, N, K)
    import torch
    import fp4_block_scaled_elem_amd as mq
    st = torch.cuda.Stream()
    xb = to_dev_bf16(workloads.random_bf16((M, K), M + K, 1.0, "lognormal_mixed"))
    wb = to_dev_bf16(workloads.random_bf16((N, K), N + K, 0.02))
    st.wait_stream(torch.cuda.current_stream())  # the inputs were copied on the default stream
    with torch.cuda.stream(st):
        qa, ga = _nvfp4(M, K)
        qw, gw = _nvfp4(N, K)
        mq.mq_quantize_nvfp4(xb, qa, stream=st)
        mq.mq_quantize_nvfp4(wb, qw, stream=st)
        outs = {}
        for name, f32 in (("bf16", False), ("f32", True)):
            c = Guarded((M, N), torch.float32 if f32 else torch.bfloat16, fill=0xFF)
            mq.mq_gemm_nvfp4_prefill(qa, None, qw, c.t, mq.MQ_OUT_F32 if f32 else 0, stream=st)
            outs[name] = c
        # fused: per-tile form, and the quantize-once form writing A's NVFP4
        cf = Guarded((M, N), torch.bfloat16, fill=0xFF)
        rec = Guarded((mq.REC_BYTES // 4,), torch.int32, fill=0)
        mq.mq_gemm_nvfp4_prefill(mq.NVFP4(None, None, rec.t), xb, qw, cf.t, mq.MQ_A_FUSED_BF16, stream=st)
        kp, gk = _nvfp4(M, K)
        cp = Guarded((M, N), torch.bfloat16, fill=0xFF)
        mq.mq_gemm_nvfp4_prefill(kp, xb, qw, cp.t, mq.MQ_A_FUSED_BF16, stream=st)
        # grouped: two weights of different row counts
        qw2, gw2 = _nvfp4(N + 7, K)
        mq.mq_quantize_nvfp4(to_dev_bf16(workloads.random_bf16((N + 7, K), 5, 0.02)), qw2, stream=st)
        g1 = Guarded((M, N), torch.bfloat16, fill=0xFF)
        g2 = Guarded((M, N + 7), torch.bfloat16, fill=0xFF)
        mq.mq_gemm_nvfp4_prefill_grouped(qa, None, [qw, qw2], [g1.t, g2.t], stream=st)
    st.synchronize()
    guards = list(ga) + list(gw) + list(gk) + list(gw2) + [rec, cf, cp, g1, g2] + list(outs.values())
    assert _all_intact(guards), "a guard byte changed"
    for c in list(outs.values()) + [cf, cp, g1, g2]:
        assert c.written(), "an output element was not written"
    assert torch.equal(outs["bf16"].t.view(torch.int16), cf.t.view(torch.int16))
    assert torch.equal(outs["bf16"].t.view(torch.int16), cp.t.view(torch.int16))
    assert torch.equal(outs["bf16"].t.view(torch.int16), g1.t.view(torch.int16))
    assert torch.equal(kp.codes, qa.codes) and torch.equal(kp.scales, qa.scales)


@pytest.mark.parametrize("M,N,K", [(1, 17, 128), (17, 1000, 4112), (32, 33, 640), (5, 4100, 256), (24, 8200, 256)])
def test_decode_paths_stay_inside_their_buffers(M, N, K):
    announce("guards decode", M, N, K)
    import torch
    import fp4_block_scaled_elem_amd as mq
    st = torch.cuda.Stream()
    x = to_dev_bf16(workloads.random_bf16((M, K), 7 + M, 1.0))
    w1 = to_dev_bf16(workloads.random_bf16((N, K), 8 + N, 0.02))
    w2 = to_dev_bf16(workloads.random_bf16((N // 2 + 1, K), 9, 0.02))
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        y = Guarded((M, N), torch.bfloat16, fill=0xFF)
        mq.mq_gemv_bf16_decode(x, w1, y.t, stream=st)
        ya = Guarded((M, N), torch.bfloat16, fill=0xFF)
        yb = Guarded((M, N // 2 + 1), torch.bfloat16, fill=0xFF)
        mq.mq_gemv_bf16_decode_grouped(x, [w1, w2], [ya.t, yb.t], stream=st)
        xq, gx = _nvfp4(M, K)
        wq, gwq = _nvfp4(N, K)
        mq.mq_quantize_nvfp4(x, xq, stream=st)
        mq.mq_quantize_nvfp4(w1, wq, stream=st)
        yq = Guarded((M, N), torch.bfloat16, fill=0xFF)
        mq.mq_gemv_nvfp4_decode(xq, wq, yq.t, stream=st)
    st.synchronize()
    assert _all_intact([y, ya, yb, yq] + list(gx) + list(gwq)), "a guard byte changed"
    assert y.written() and ya.written() and yb.written() and yq.written()
    assert torch.equal(y.t.view(torch.int16), ya.t.view(torch.int16))


@pytest.mark.parametrize("rows,cols", [(7, 48), (300, 1040)])
def test_producers_stay_inside_their_buffers(rows, cols):
    announce("guards producers", rows, cols)
    import torch
    import fp4_block_scaled_elem_amd as mq
    st = torch.cuda.Stream()
    x = to_dev_bf16(workloads.random_bf16((rows, cols), 3, 1.0))
    g = to_dev_bf16(workloads.random_bf16((cols,), 4, 1.0))
    b = to_dev_bf16(workloads.random_bf16((rows, cols), 5, 1.0))
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        y1 = Guarded((rows, cols), torch.bfloat16, fill=0xFF)
        r1 = Guarded((mq.REC_BYTES // 4,), torch.int32, fill=0)
        mq.mq_rmsnorm_amax(x, g, y1.t, r1.t, stream=st)
        y2 = Guarded((rows, cols), torch.bfloat16, fill=0xFF)
        r2 = Guarded((mq.REC_BYTES // 4,), torch.int32, fill=0)
        mq.mq_swiglu_amax(x, b, y2.t, r2.t, stream=st)
    st.synchronize()
    assert _all_intact([y1, r1, y2, r2]), "a guard byte changed"
    assert y1.written() and y2.written()


@pytest.mark.parametrize("M", [3, 70])
def test_linear_stays_inside_its_buffers(M):
    announce("guards linear", M)
    import torch
    import fp4_block_scaled_elem_amd as mq
    st = torch.cuda.Stream()
    N, K = 300, 512
    with torch.cuda.stream(st):
        wn, gwn = _nvfp4(N, K)
        lin = mq.Linear(to_dev_bf16(workloads.random_bf16((N, K), 11, 0.02)))
        lin.w_nvfp4 = wn
        lin.prepare(stream=st)
        x = to_dev_bf16(workloads.random_bf16((M, K), 12, 1.0))
        aw, gaw = _nvfp4(M, K)
        y = Guarded((M, N), torch.bfloat16, fill=0xFF)
        lin.forward(x, out=y.t, a_work=aw, stream=st)
    st.synchronize()
    assert _all_intact([y] + list(gwn) + list(gaw)), "a guard byte changed"
    assert y.written()
