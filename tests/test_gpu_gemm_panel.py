"""GPU parity of the fused prologue's quantize-once form.

With MQ_A_FUSED_BF16 and A's codes and scale buffers given, every workgroup
quantizes the 256-row panel of A its tiles read into those buffers, then
multiplies from them (shapes outside the direct-copy path: the standalone
encode pass into the same buffers, then the plain GEMM).  Both must leave
exactly the bytes mq_quantize_nvfp4 writes (codes, scale bytes, s_t) and a C
bit-identical to the two-kernel path (quantize, then the GEMM), which the
other GEMM tests hold to the float64 oracle; small cases are checked
against the oracle here too.  Shapes cover one tile per workgroup, several
panels with a ragged last one, the loop over several column tiles per
workgroup (M = 32768: two workgroups per panel), ragged K (the fallback),
grouped launches, a given tensor scale and a producer's partial maxima.

By default the library takes the panel form only where each workgroup of a
panel gets at least four column tiles (M of about 16384 and more); these
tests lower that threshold to one tile (a test-support knob) so that the
panel kernel runs at their small shapes, and one test checks the default
routing of a small panel count (the separate path) against the forced panel
form, bit for bit.
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


@pytest.fixture(autouse=True)
def _panel_form_everywhere():
    mq = _mq()
    old = mq.mq_check_set_panel_min_tiles(1)
    yield
    mq.mq_check_set_panel_min_tiles(old)


def _run_panel(x, ws, M, f32=False, flags=0, a=None):
    """Fused launch with A's buffers given; returns (outputs, a)."""
    import torch
    mq = _mq()
    K = x.shape[1]
    a = a if a is not None else mq.NVFP4.empty(M, K)
    dt = torch.float32 if f32 else torch.bfloat16
    cs = [torch.empty((M, w.shape[0]), dtype=dt, device="cuda") for w in ws]
    f = mq.MQ_A_FUSED_BF16 | flags | (mq.MQ_OUT_F32 if f32 else 0)
    if len(ws) == 1:
        mq.mq_gemm_nvfp4_prefill(a, x, ws[0], cs[0], f)
    else:
        mq.mq_gemm_nvfp4_prefill_grouped(a, x, ws, cs, f)
    torch.cuda.synchronize()
    return cs, a


def _run_plain(qa, ws, M, f32=False):
    import torch
    mq = _mq()
    dt = torch.float32 if f32 else torch.bfloat16
    cs = []
    for w in ws:
        c = torch.empty((M, w.shape[0]), dtype=dt, device="cuda")
        mq.mq_gemm_nvfp4_prefill(qa, None, w, c, mq.MQ_OUT_F32 if f32 else 0)
        cs.append(c)
    torch.cuda.synchronize()
    return cs


def _same(a, b):
    import torch
    v = torch.int32 if a.dtype == torch.float32 else torch.int16
    return torch.equal(a.view(v), b.view(v))


def _same_quantization(a, qa):
    c1, s1, t1 = quantized_host(a)
    c2, s2, t2 = quantized_host(qa)
    return t1 == t2 and np.array_equal(s1, s2) and np.array_equal(c1, c2)


@pytest.mark.parametrize("M,N,K,seed", [(300, 520, 512, 0), (700, 1300, 1024, 1), (100, 300, 272, 2),
                                        (64, 256, 4112, 3)])
def test_panel_bit_identical_to_two_kernels(M, N, K, seed):
    announce("gemm panel vs two kernels", M, N, K)
    mq = _mq()
    xa = workloads.random_bf16((M, K), seed, 1.0, "lognormal_mixed")
    xw = workloads.random_bf16((N, K), seed + 50, 0.02)
    x = to_dev_bf16(xa)
    qw = mq.quantize(to_dev_bf16(xw))
    qa = mq.quantize(x)
    for f32 in (False, True):
        (c_pan,), a = _run_panel(x, [qw], M, f32=f32)
        (c_two,) = _run_plain(qa, [qw], M, f32=f32)
        assert _same(c_pan, c_two), f"f32={f32}: output differs"
        assert _same_quantization(a, qa), f"f32={f32}: A's NVFP4 differs"
    # and the oracle (quantization bytes and the bf16 output)
    oa = oracle.quantize_nvfp4(xa)
    codes, scales, st = quantized_host(a)
    assert st == int(np.float32(oa.s_t).view(np.uint32))
    assert np.array_equal(scales, oa.scales) and np.array_equal(codes, oa.codes)
    (c_bf,), _ = _run_panel(x, [qw], M)
    r = rule_t(bf16_dev_to_f64(c_bf), oracle.gemm_nvfp4_ref(oa, oracle.quantize_nvfp4(xw)), bf16_out=True)
    print("  rule T:", r, flush=True)
    assert r.ok, str(r)


def test_panel_loops_over_column_tiles():
    # M = 32768: 128 panels, two workgroups per panel on 256 CUs, each taking
    # every other one of the four column tiles
    announce("gemm panel, several column tiles per workgroup")
    import torch
    mq = _mq()
    M, N, K = 32768, 1024, 256
    xa = workloads.random_bf16((M, K), 7, 1.0, "lognormal_mixed")
    xw = workloads.random_bf16((N, K), 8, 0.02)
    x = to_dev_bf16(xa)
    qw = mq.quantize(to_dev_bf16(xw))
    qa = mq.quantize(x)
    (c_pan,), a = _run_panel(x, [qw], M)
    (c_two,) = _run_plain(qa, [qw], M)
    assert _same(c_pan, c_two)
    assert _same_quantization(a, qa)
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([rng.choice(M, 128, replace=False), [0, 255, 256, M - 1]]))
    oa = oracle.quantize_nvfp4(xa, rows=rows)
    ref = oracle.gemm_nvfp4_ref(oa, oracle.quantize_nvfp4(xw))
    r = rule_t(bf16_dev_to_f64(c_pan[torch.from_numpy(rows).cuda()]), ref, bf16_out=True)
    print("  rule T (sampled rows):", r, flush=True)
    assert r.ok, str(r)


@pytest.mark.parametrize("M,Ns,K", [(600, (512, 300), 512), (260, (256, 1024, 72), 272)])
def test_panel_grouped_bit_identical(M, Ns, K):
    announce("gemm panel grouped", M, Ns, K)
    mq = _mq()
    xa = workloads.random_bf16((M, K), 11, 1.0, "lognormal_mixed")
    x = to_dev_bf16(xa)
    ws = [mq.quantize(to_dev_bf16(workloads.random_bf16((n, K), 12 + i, 0.02))) for i, n in enumerate(Ns)]
    qa = mq.quantize(x)
    cs, a = _run_panel(x, ws, M)
    ref = _run_plain(qa, ws, M)
    for g, (c1, c2) in enumerate(zip(cs, ref)):
        assert _same(c1, c2), f"group {g}"
    assert _same_quantization(a, qa)


def test_panel_given_scale():
    announce("gemm panel given scale")
    import torch
    mq = _mq()
    M, N, K = 300, 256, 512
    xa = workloads.random_bf16((M, K), 21, 3.0)
    x = to_dev_bf16(xa)
    qw = mq.quantize(to_dev_bf16(workloads.random_bf16((N, K), 22, 0.02)))
    a = mq.NVFP4.empty(M, K)
    a.set_s_t(0.0078125)
    (c,), a = _run_panel(x, [qw], M, flags=mq.MQ_SCALE_GIVEN, a=a)
    qa = mq.NVFP4.empty(M, K)
    qa.set_s_t(0.0078125)
    mq.mq_quantize_nvfp4(x, qa, mq.MQ_SCALE_GIVEN)
    (c2,) = _run_plain(qa, [qw], M)
    torch.cuda.synchronize()
    assert _same(c, c2) and _same_quantization(a, qa)
    oa = oracle.quantize_nvfp4(xa, s_t=np.float32(0.0078125))
    codes, scales, _ = quantized_host(a)
    assert np.array_equal(codes, oa.codes) and np.array_equal(scales, oa.scales)


def test_panel_from_producer_partials():
    announce("gemm panel from rmsnorm partials")
    import torch
    mq = _mq()
    M, N, K = 512, 512, 1024
    xb = workloads.random_bf16((M, K), 31, 1.0, "lognormal_mixed")
    gb = workloads.random_bf16((K,), 32, 1.0)
    y = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    a = mq.NVFP4.empty(M, K)
    mq.mq_rmsnorm_amax(to_dev_bf16(xb), to_dev_bf16(gb), y, a.rec)
    qw = mq.quantize(to_dev_bf16(workloads.random_bf16((N, K), 33, 0.02)))
    (c,), a = _run_panel(y, [qw], M, flags=mq.MQ_SCALE_PARTIALS, a=a)
    qa = mq.quantize(y)
    (c2,) = _run_plain(qa, [qw], M)
    assert _same(c, c2) and _same_quantization(a, qa)


def test_linear_fused_with_work_buffers_takes_the_panel_form():
    # the phase-aware linear's fused prefill with a full NVFP4 work buffer
    # routes to the quantize-once form: same output as the plain path, and
    # the work buffer ends up holding x's NVFP4
    announce("linear fused with work buffers")
    import torch
    mq = _mq()
    M, K, N = 300, 1024, 512
    lin = mq.Linear(to_dev_bf16(workloads.random_bf16((N, K), 41, 0.02))).prepare()
    x = to_dev_bf16(workloads.random_bf16((M, K), 42, 1.0, "lognormal_mixed"))
    aw = mq.NVFP4.empty(M, K)
    y = lin.forward(x, flags=mq.MQ_A_FUSED_BF16, a_work=aw)
    y2 = lin.forward(x)
    qa = mq.quantize(x)
    torch.cuda.synchronize()
    assert _same(y, y2)
    assert _same_quantization(aw, qa)


@pytest.mark.parametrize("M,Ns,K", [(256, (4096,), 4096), (1000, (520, 300), 1024)])
def test_default_routing_matches_forced_panel_form(M, Ns, K):
    # one or two 256-row panels: with the default threshold the call takes
    # the encode pass and the plain GEMM (far faster there); its output and
    # A's bytes equal the forced panel form's and the standalone quantizer's
    announce("panel threshold: default vs forced", M, Ns, K)
    mq = _mq()
    x = to_dev_bf16(workloads.random_bf16((M, K), 90 + M, 1.0, "lognormal_mixed"))
    ws = [mq.quantize(to_dev_bf16(workloads.random_bf16((n, K), 91 + g, 0.02))) for g, n in enumerate(Ns)]
    cs_forced, a_forced = _run_panel(x, ws, M)
    old = mq.mq_check_set_panel_min_tiles(4)
    try:
        cs_default, a_default = _run_panel(x, ws, M)
    finally:
        mq.mq_check_set_panel_min_tiles(old)
    qa = mq.quantize(x)
    assert all(_same(c1, c2) for c1, c2 in zip(cs_forced, cs_default))
    assert _same_quantization(a_forced, qa) and _same_quantization(a_default, qa)
