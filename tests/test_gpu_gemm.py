"""GPU parity of mq_gemm_nvfp4_prefill against the float64 oracle.

Outputs are compared element by element with the stated tolerance (rule T
in tests/parity.py); the binary32 output mode is checked against the
literal criterion.  The fused (bf16 A, quantized in the GEMM) path must give
bit-identical results to quantize-then-GEMM.
"""

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import announce, bf16_dev_to_f64, to_dev_bf16, upload_nvfp4
from tests.parity import rule_t

pytestmark = pytest.mark.gpu


def _mq():
    import fp4_block_scaled_elem_amd as mq
    return mq


def _gemm(qa, qw, M, N, f32=False, stream=None):
    import torch
    mq = _mq()
    c = torch.empty((M, N), dtype=torch.float32 if f32 else torch.bfloat16, device="cuda")
    mq.mq_gemm_nvfp4_prefill(qa, None, qw, c, mq.MQ_OUT_F32 if f32 else 0, stream)
    torch.cuda.synchronize()
    return c


def _out(c):
    import torch
    if c.dtype == torch.float32:
        return c.cpu().numpy().astype(np.float64)
    return bf16_dev_to_f64(c)


def _assert_rule_t(got, ref, bf16):
    r = rule_t(got, ref, bf16_out=bf16)
    print("  rule T:", r, flush=True)
    assert r.ok, str(r)


@pytest.mark.parametrize("M,N,K,seed", [
    (1, 1, 16, 0), (37, 53, 48, 1), (100, 200, 144, 2), (300, 260, 4112, 3),
    (257, 129, 512, 4), (64, 1000, 256, 5), (512, 512, 1024, 6), (33, 300, 2064, 7),
])
def test_ragged_shapes_uploaded_operands(M, N, K, seed):
    announce("gemm ragged", M, N, K, seed)
    xa = workloads.random_bf16((M, K), seed, 1.0, "normal")
    xw = workloads.random_bf16((N, K), seed + 50, 0.02, "normal")
    oa, ow = oracle.quantize_nvfp4(xa), oracle.quantize_nvfp4(xw)
    ref = oracle.gemm_nvfp4_ref(oa, ow)
    qa, qw = upload_nvfp4(oa), upload_nvfp4(ow)
    _assert_rule_t(_out(_gemm(qa, qw, M, N)), ref, True)
    _assert_rule_t(_out(_gemm(qa, qw, M, N, f32=True)), ref, False)


def test_identity_weight_is_exact_in_f32_mode():
    # W = 2688 I: every output is one product g*sigma*2688 times s_tA, so the
    # binary32 output is the binary32 rounding of the exact oracle value;
    # any transposed or shifted index shows up as a mismatch
    announce("gemm identity weight")
    K = 256
    xa = workloads.random_bf16((96, K), 11, 1.0, "lognormal_mixed")
    w = workloads.f32_to_bf16_bits(np.eye(K, dtype=np.float32) * np.float32(2688.0))
    oa, ow = oracle.quantize_nvfp4(xa), oracle.quantize_nvfp4(w)
    ref = oracle.gemm_nvfp4_ref(oa, ow)
    got = _out(_gemm(upload_nvfp4(oa), upload_nvfp4(ow), 96, K, f32=True))
    assert np.array_equal(got, ref.astype(np.float32).astype(np.float64))


def test_cfg1_end_to_end_and_determinism():
    announce("gemm cfg1 end to end")
    import torch
    mq = _mq()
    xa, xw = workloads.activation(1), workloads.weight(1)
    qa, qw = mq.quantize(to_dev_bf16(xa)), mq.quantize(to_dev_bf16(xw))
    ref = oracle.gemm_nvfp4_ref(oracle.quantize_nvfp4(xa), oracle.quantize_nvfp4(xw))
    c1 = _gemm(qa, qw, 128, 512)
    _assert_rule_t(_out(c1), ref, True)
    _assert_rule_t(_out(_gemm(qa, qw, 128, 512, f32=True)), ref, False)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c2 = torch.empty_like(c1)
        mq.mq_gemm_nvfp4_prefill(qa, None, qw, c2, 0, s)
    s.synchronize()
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))


def _fused(x_dev, qw, M, N, f32=False):
    import torch
    mq = _mq()
    c = torch.empty((M, N), dtype=torch.float32 if f32 else torch.bfloat16, device="cuda")
    a = mq.NVFP4(None, None, torch.zeros(mq.REC_BYTES // 4, dtype=torch.int32, device="cuda"))
    mq.mq_gemm_nvfp4_prefill(a, x_dev, qw, c, mq.MQ_A_FUSED_BF16 | (mq.MQ_OUT_F32 if f32 else 0))
    torch.cuda.synchronize()
    return c, a


@pytest.mark.parametrize("M,N,K,seed", [(128, 512, 512, 0), (37, 300, 4112, 1), (500, 260, 1024, 2)])
def test_fused_prologue_bit_identical_to_unfused(M, N, K, seed):
    announce("gemm fused vs unfused", M, N, K)
    import torch
    mq = _mq()
    xa = workloads.random_bf16((M, K), seed, 1.0, "lognormal_mixed")
    xw = workloads.random_bf16((N, K), seed + 9, 0.02)
    x = to_dev_bf16(xa)
    qw = mq.quantize(to_dev_bf16(xw))
    qa = mq.quantize(x)
    for f32 in (False, True):
        c_unf = _gemm(qa, qw, M, N, f32=f32)
        c_fus, a = _fused(x, qw, M, N, f32=f32)
        assert torch.equal(c_unf.view(torch.int32 if f32 else torch.int16),
                           c_fus.view(torch.int32 if f32 else torch.int16))
        assert a.s_t() == qa.s_t()
    ref = oracle.gemm_nvfp4_ref(oracle.quantize_nvfp4(xa), oracle.quantize_nvfp4(xw))
    _assert_rule_t(_out(c_unf), ref, False)


@pytest.mark.parametrize("K", [256, 272])
def test_fused_prologue_reciprocal_overflow(K):
    # activations of bf16 subnormals only: s_tA is so small that every
    # reciprocal group scale overflows to +inf, where zero elements keep a
    # sign-only code and the others saturate (the quantizer's fix-up path,
    # compiled separately from the common one); large weights keep the
    # output scale s_tA*s_tW normal, so a wrong code shows in the output
    announce("gemm fused reciprocal overflow", K)
    import torch
    mq = _mq()
    M, N = 64, 128
    rng = np.random.default_rng(31 + K)
    xa = np.zeros((M, K), np.uint16)
    xa[rng.random((M, K)) < 0.3] = 0x8000                       # -0
    nz = rng.random((M, K)) < 0.2
    xa[nz] = rng.integers(1, 8, int(nz.sum())).astype(np.uint16) | \
        np.where(rng.random(int(nz.sum())) < 0.5, 0x8000, 0).astype(np.uint16)
    xw = workloads.random_bf16((N, K), 33, 1.0e37)
    x = to_dev_bf16(xa)
    qw = mq.quantize(to_dev_bf16(xw))
    qa = mq.quantize(x)
    oa = oracle.quantize_nvfp4(xa)
    assert np.array_equal(qa.codes.cpu().numpy().reshape(oa.codes.shape), oa.codes)
    c_unf = _gemm(qa, qw, M, N, f32=True)
    c_fus, a = _fused(x, qw, M, N, f32=True)
    assert torch.equal(c_unf.view(torch.int32), c_fus.view(torch.int32))
    assert a.s_t() == qa.s_t()
    ref = oracle.gemm_nvfp4_ref(oa, oracle.quantize_nvfp4(xw))
    assert np.abs(ref).max() > 0
    _assert_rule_t(_out(c_fus), ref, False)


def test_fused_given_scale():
    announce("gemm fused given scale")
    import torch
    mq = _mq()
    M, N, K = 64, 128, 256
    xa = workloads.random_bf16((M, K), 21, 3.0)
    xw = workloads.random_bf16((N, K), 22, 0.02)
    qw = mq.quantize(to_dev_bf16(xw))
    a = mq.NVFP4(None, None, torch.zeros(mq.REC_BYTES // 4, dtype=torch.int32, device="cuda"))
    a.set_s_t(0.0078125)
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mq.mq_gemm_nvfp4_prefill(a, to_dev_bf16(xa), qw, c, mq.MQ_A_FUSED_BF16 | mq.MQ_SCALE_GIVEN)
    torch.cuda.synchronize()
    ref = oracle.gemm_nvfp4_ref(oracle.quantize_nvfp4(xa, s_t=np.float32(0.0078125)),
                                oracle.quantize_nvfp4(xw))
    _assert_rule_t(_out(c), ref, True)


def _sampled_projection(cfg, proj, nrows=256, ncols=512, fused=False):
    import torch
    mq = _mq()
    c = workloads.CONFIGS[cfg]
    act = workloads.PROJ_INPUT[proj]
    xa = workloads.activation(cfg, act)
    xw = workloads.weight(cfg, proj)
    M, K = xa.shape
    N = xw.shape[0]
    x = to_dev_bf16(xa)
    qw = mq.quantize(to_dev_bf16(xw))
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    if fused:
        a = mq.NVFP4(None, None, torch.zeros(mq.REC_BYTES // 4, dtype=torch.int32, device="cuda"))
        mq.mq_gemm_nvfp4_prefill(a, x, qw, out, mq.MQ_A_FUSED_BF16)
    else:
        qa = mq.quantize(x)
        mq.mq_gemm_nvfp4_prefill(qa, None, qw, out, 0)
    torch.cuda.synchronize()
    rng = np.random.default_rng([cfg, len(proj)])
    rows = np.unique(np.concatenate([rng.choice(M, nrows, replace=False), [0, M - 1]]))
    cols = np.unique(np.concatenate([rng.choice(N, min(ncols, N), replace=False), [0, N - 1]]))
    oa = oracle.quantize_nvfp4(xa, rows=rows)
    ow = oracle.quantize_nvfp4(xw, rows=cols)
    ref = oracle.gemm_nvfp4_ref(oa, ow)
    got = bf16_dev_to_f64(out[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()])
    _assert_rule_t(got, ref, True)


@pytest.mark.parametrize("proj", workloads.PROJS)
def test_cfg2_projection_sampled(proj):
    announce("gemm cfg2 sampled", proj)
    _sampled_projection(2, proj)


@pytest.mark.parametrize("proj", ["k", "down"])
def test_cfg3_fused_projection_sampled(proj):
    announce("gemm cfg3 fused sampled", proj)
    _sampled_projection(3, proj, fused=True)


@pytest.mark.parametrize("proj", ["k", "gate", "down"])
def test_cfg5_projection_sampled(proj):
    announce("gemm cfg5 sampled", proj)
    _sampled_projection(5, proj)


@pytest.mark.parametrize("M,N,K", [(256, 512, 1024), (300, 260, 4112), (64, 1003, 512)])
def test_bf16_output_is_nearest_even_rounding_of_f32_output(M, N, K):
    # kernel property (no oracle involved): the bf16 mode stores exactly the
    # round-to-nearest-even of what the binary32 mode stores
    announce("gemm bf16 == rne(f32)", M, N, K)
    import torch
    mq = _mq()
    qa = mq.quantize(to_dev_bf16(workloads.random_bf16((M, K), 31, 1.0, "lognormal_mixed")))
    qw = mq.quantize(to_dev_bf16(workloads.random_bf16((N, K), 32, 0.02)))
    c32 = _gemm(qa, qw, M, N, f32=True).cpu().numpy()
    c16 = _gemm(qa, qw, M, N).view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(c16, workloads.f32_to_bf16_bits(c32))


def _grouped(qa, x, ws, M, f32=False):
    import torch
    mq = _mq()
    dt = torch.float32 if f32 else torch.bfloat16
    cs = [torch.empty((M, w.shape[0]), dtype=dt, device="cuda") for w in ws]
    flags = mq.MQ_OUT_F32 if f32 else 0
    if x is not None:
        flags |= mq.MQ_A_FUSED_BF16
    mq.mq_gemm_nvfp4_prefill_grouped(qa, x, ws, cs, flags)
    torch.cuda.synchronize()
    return cs


@pytest.mark.parametrize("M,Ns,K,seed", [
    (300, (100, 260, 64), 512, 0),          # ragged groups, K % 128 == 0
    (130, (512, 33), 4112, 1),               # ragged K
    (257, (1024, 1024, 256, 16), 1024, 2),   # four groups
    (64, (700,), 256, 3),                    # one group
])
def test_grouped_bit_identical_to_single_calls(M, Ns, K, seed):
    # each output of the grouped launch must equal the single-weight call bit
    # for bit (every element is accumulated in the same order whatever the
    # tile shape); one group is also checked against the oracle
    announce("gemm grouped vs single", M, Ns, K, seed)
    import torch
    mq = _mq()
    xa = workloads.random_bf16((M, K), seed, 1.0, "lognormal_mixed")
    xws = [workloads.random_bf16((n, K), seed + 20 + i, 0.02) for i, n in enumerate(Ns)]
    x = to_dev_bf16(xa)
    qa = mq.quantize(x)
    ws = [mq.quantize(to_dev_bf16(xw)) for xw in xws]
    for f32 in (False, True):
        view = torch.int32 if f32 else torch.int16
        cs = _grouped(qa, None, ws, M, f32)
        for w, c in zip(ws, cs):
            assert torch.equal(c.view(view), _gemm(qa, w, M, w.shape[0], f32=f32).view(view))
        fs = _grouped(mq.NVFP4(None, None, torch.zeros(mq.REC_BYTES // 4, dtype=torch.int32, device="cuda")),
                      x, ws, M, f32)
        for c, f in zip(cs, fs):
            assert torch.equal(c.view(view), f.view(view))
    ref = oracle.gemm_nvfp4_ref(oracle.quantize_nvfp4(xa), oracle.quantize_nvfp4(xws[-1]))
    _assert_rule_t(_out(cs[-1]), ref, False)


def test_cfg2_grouped_gate_up_sampled():
    # the launch the 8B-shape benchmark uses for the MLP input projections
    announce("gemm cfg2 grouped gate+up")
    import torch
    mq = _mq()
    xa = workloads.activation(2, "x_gu")
    M, K = xa.shape
    xws = [workloads.weight(2, p) for p in ("gate", "up")]
    qa = mq.quantize(to_dev_bf16(xa))
    ws = [mq.quantize(to_dev_bf16(xw)) for xw in xws]
    cs = _grouped(qa, None, ws, M)
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([rng.choice(M, 192, replace=False), [0, M - 1]]))
    oa = oracle.quantize_nvfp4(xa, rows=rows)
    for xw, c in zip(xws, cs):
        N = xw.shape[0]
        cols = np.unique(np.concatenate([rng.choice(N, 384, replace=False), [0, N - 1]]))
        ref = oracle.gemm_nvfp4_ref(oa, oracle.quantize_nvfp4(xw, rows=cols))
        got = bf16_dev_to_f64(c[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()])
        _assert_rule_t(got, ref, True)


@pytest.mark.parametrize("M,K", [(256, 512), (128, 1024), (255, 512), (257, 512), (64, 4096)])
def test_fused_inline_amax_boundary(M, K):
    # the per-tile fused form takes max|A| inside the GEMM when M*K <= 2^17
    # (one launch) and runs the amax pass otherwise; the largest magnitude is
    # planted in the last element, which the in-GEMM maximum must reach; both
    # sides of the limit must match quantize-then-GEMM bit for bit
    announce("gemm fused inline amax", M, K)
    import torch
    mq = _mq()
    N = 300
    xa = workloads.random_bf16((M, K), 71 + M, 1.0, "normal")
    xa[-1, -1] = workloads.f32_to_bf16_bits(np.array([-1000.0], np.float32))[0]
    xw = workloads.random_bf16((N, K), 72, 0.02)
    x = to_dev_bf16(xa)
    qw = mq.quantize(to_dev_bf16(xw))
    qa = mq.quantize(x)
    c_unf = _gemm(qa, qw, M, N, f32=True)
    c_fus, a = _fused(x, qw, M, N, f32=True)
    assert torch.equal(c_unf.view(torch.int32), c_fus.view(torch.int32))
    rec = a.rec.cpu().numpy().view(np.uint32)
    ref = oracle.quantize_nvfp4(xa)
    assert int(rec[0]) == int(np.float32(ref.s_t).view(np.uint32))
    assert int(rec[1]) == (int(xa[-1, -1]) & 0x7FFF) << 16
    _assert_rule_t(_out(c_fus), oracle.gemm_nvfp4_ref(ref, oracle.quantize_nvfp4(xw)), False)
