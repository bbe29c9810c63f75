"""GPU parity of the small-problem GEMM kernel (M <= 128 rows of A).

Below 129 rows every A form of mq_gemm_nvfp4_prefill (packed A, bf16 A
quantized in the launch, and the quantize-once form that also stores A's
NVFP4) runs one kernel that splits K over its waves.  Its outputs are held
to the float64 oracle under rule T (tests/parity.py) and, in binary32
mode, to the literal criterion; the A forms, groupings and streams must
agree bit for bit; the NVFP4 the quantize-once form stores must equal the
oracle's bytes.  The row-count boundary (128 / 129) is covered on both
sides.
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


def _c(M, N, f32):
    import torch
    return torch.full((M, N), float("nan"), dtype=torch.float32 if f32 else torch.bfloat16, device="cuda")


def _out(c):
    import torch
    if c.dtype == torch.float32:
        return c.cpu().numpy().astype(np.float64)
    return bf16_dev_to_f64(c)


def _bits(c):
    import torch
    return c.view(torch.int32 if c.dtype == torch.float32 else torch.int16)


def _rule_t(got, ref, bf16):
    r = rule_t(got, ref, bf16_out=bf16)
    print("  rule T:", r, flush=True)
    assert r.ok, str(r)


def _rec():
    import torch
    mq = _mq()
    return torch.zeros(mq.REC_BYTES // 4, dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("M,N,K,seed", [
    (1, 16, 128, 0), (1, 300, 4096, 1), (5, 77, 512, 2), (16, 512, 512, 3), (17, 129, 1024, 4),
    (32, 1000, 256, 5), (100, 260, 4112, 6), (128, 512, 512, 7), (128, 1024, 14336, 8), (64, 33, 16, 9),
    (127, 200, 272, 10),
])
def test_small_against_oracle_every_form(M, N, K, seed):
    announce("gemm small", M, N, K, seed)
    import torch
    mq = _mq()
    xa = workloads.random_bf16((M, K), seed, 1.0, "lognormal_mixed")
    xw = workloads.random_bf16((N, K), seed + 40, 0.02)
    oa, ow = oracle.quantize_nvfp4(xa), oracle.quantize_nvfp4(xw)
    ref = oracle.gemm_nvfp4_ref(oa, ow)
    qa, qw = upload_nvfp4(oa), upload_nvfp4(ow)
    x = to_dev_bf16(xa)
    for f32 in (False, True):
        flags = mq.MQ_OUT_F32 if f32 else 0
        c_packed = _c(M, N, f32)
        mq.mq_gemm_nvfp4_prefill(qa, None, qw, c_packed, flags)
        c_fused = _c(M, N, f32)
        a_f = mq.NVFP4(None, None, _rec())
        mq.mq_gemm_nvfp4_prefill(a_f, x, qw, c_fused, flags | mq.MQ_A_FUSED_BF16)
        c_once = _c(M, N, f32)
        a_once = mq.NVFP4.empty(M, K)
        mq.mq_gemm_nvfp4_prefill(a_once, x, qw, c_once, flags | mq.MQ_A_FUSED_BF16)
        torch.cuda.synchronize()
        assert torch.equal(_bits(c_packed), _bits(c_fused)), "fused A differs from packed A"
        assert torch.equal(_bits(c_packed), _bits(c_once)), "quantize-once form differs from packed A"
        assert a_f.s_t() == np.float32(oa.s_t) and a_once.s_t() == np.float32(oa.s_t)
        assert np.array_equal(a_once.codes.cpu().numpy(), oa.codes), "stored A codes differ from the oracle"
        assert np.array_equal(a_once.scales.cpu().numpy(), oa.scales), "stored A scales differ from the oracle"
        _rule_t(_out(c_packed), ref, not f32)


@pytest.mark.parametrize("M", [128, 129])
def test_row_boundary_both_sides(M):
    # 128 rows take the small kernel, 129 the tiled one: both within rule T,
    # and each bit-identical across its A forms
    announce("gemm small boundary", M)
    import torch
    mq = _mq()
    N, K = 384, 1024
    xa = workloads.random_bf16((M, K), 300 + M, 1.0, "normal")
    xw = workloads.random_bf16((N, K), 301, 0.02)
    oa, ow = oracle.quantize_nvfp4(xa), oracle.quantize_nvfp4(xw)
    qa, qw = upload_nvfp4(oa), upload_nvfp4(ow)
    c1, c2 = _c(M, N, True), _c(M, N, True)
    mq.mq_gemm_nvfp4_prefill(qa, None, qw, c1, mq.MQ_OUT_F32)
    mq.mq_gemm_nvfp4_prefill(mq.NVFP4(None, None, _rec()), to_dev_bf16(xa), qw, c2,
                             mq.MQ_OUT_F32 | mq.MQ_A_FUSED_BF16)
    torch.cuda.synchronize()
    assert torch.equal(_bits(c1), _bits(c2))
    _rule_t(_out(c1), oracle.gemm_nvfp4_ref(oa, ow), False)


@pytest.mark.parametrize("M,Ns,K", [(40, (512, 128, 128), 512), (128, (1024, 300, 16), 272), (7, (4096,), 4096)])
def test_small_grouped_bit_identical_to_single_calls(M, Ns, K):
    announce("gemm small grouped", M, Ns, K)
    import torch
    mq = _mq()
    xa = workloads.random_bf16((M, K), 500 + M, 1.0, "lognormal_mixed")
    x = to_dev_bf16(xa)
    oa = oracle.quantize_nvfp4(xa)
    qa = upload_nvfp4(oa)
    ows = [oracle.quantize_nvfp4(workloads.random_bf16((n, K), 510 + g, 0.02)) for g, n in enumerate(Ns)]
    qws = [upload_nvfp4(o) for o in ows]
    cs = [_c(M, n, False) for n in Ns]
    mq.mq_gemm_nvfp4_prefill_grouped(mq.NVFP4(None, None, _rec()), x, qws, cs, mq.MQ_A_FUSED_BF16)
    s = torch.cuda.Stream()
    singles = []
    with torch.cuda.stream(s):
        for qw, n in zip(qws, Ns):
            c = _c(M, n, False)
            mq.mq_gemm_nvfp4_prefill(qa, None, qw, c, 0, s)
            singles.append(c)
    torch.cuda.synchronize()
    s.synchronize()
    for c, c1, ow in zip(cs, singles, ows):
        assert torch.equal(_bits(c), _bits(c1)), "grouped output differs from the single call"
        _rule_t(_out(c), oracle.gemm_nvfp4_ref(oa, ow), True)


def test_small_given_scale_and_reciprocal_overflow():
    # a given tensor scale (taken from the record, not the data), and a tiny
    # activation whose reciprocal group scales overflow: the quantizer's
    # fix-up path inside the small kernel, against the standalone quantizer
    announce("gemm small given scale / overflow")
    import torch
    mq = _mq()
    M, N, K = 48, 200, 512
    xw = workloads.random_bf16((N, K), 601, 0.02)
    qw = mq.quantize(to_dev_bf16(xw))
    # bf16 subnormals and -0 only: every reciprocal group scale overflows;
    # weights near the top of the range keep s_tA * s_tW normal
    rng = np.random.default_rng(600)
    small = np.zeros((M, K), np.uint16)
    small[rng.random((M, K)) < 0.3] = 0x8000
    nz = rng.random((M, K)) < 0.2
    small[nz] = rng.integers(1, 8, int(nz.sum())).astype(np.uint16) | \
        np.where(rng.random(int(nz.sum())) < 0.5, 0x8000, 0).astype(np.uint16)
    xw_big = workloads.random_bf16((N, K), 602, 1.0e37)
    qw_big = mq.quantize(to_dev_bf16(xw_big))
    for xa, w in ((workloads.random_bf16((M, K), 603, 1.0, "lognormal_mixed"), qw), (small, qw_big)):
        x = to_dev_bf16(xa)
        qa = mq.quantize(x)
        c_ref, c_dyn, c_giv = _c(M, N, True), _c(M, N, True), _c(M, N, True)
        mq.mq_gemm_nvfp4_prefill(qa, None, w, c_ref, mq.MQ_OUT_F32)
        mq.mq_gemm_nvfp4_prefill(mq.NVFP4(None, None, _rec()), x, w, c_dyn, mq.MQ_OUT_F32 | mq.MQ_A_FUSED_BF16)
        keep = mq.NVFP4.empty(M, K)
        keep.rec.copy_(qa.rec)  # s_t of the data, given
        mq.mq_gemm_nvfp4_prefill(keep, x, w, c_giv, mq.MQ_OUT_F32 | mq.MQ_A_FUSED_BF16 | mq.MQ_SCALE_GIVEN)
        torch.cuda.synchronize()
        assert torch.equal(_bits(c_ref), _bits(c_dyn)) and torch.equal(_bits(c_ref), _bits(c_giv))
        assert torch.equal(keep.codes, qa.codes) and torch.equal(keep.scales, qa.scales)
        oa = oracle.quantize_nvfp4(xa)
        assert np.array_equal(qa.codes.cpu().numpy(), oa.codes)
        _rule_t(_out(c_ref), oracle.gemm_nvfp4_ref(oa, oracle.quantize_nvfp4(
            xw if w is qw else xw_big)), False)


def test_cfg1_single_linear_one_launch_every_form():
    # the single linear of 128 x 512 x 512: packed, fused and quantize-once
    # forms agree bit for bit with each other and hold rule T
    announce("gemm small cfg1")
    import torch
    mq = _mq()
    xa, xw = workloads.activation(1), workloads.weight(1)
    oa, ow = oracle.quantize_nvfp4(xa), oracle.quantize_nvfp4(xw)
    qw = mq.quantize(to_dev_bf16(xw))
    x = to_dev_bf16(xa)
    y_sep = mq.prefill_linear(x, qw)
    y_fus = mq.prefill_linear(x, qw, fused=True)
    keep = mq.NVFP4.empty(128, 512)
    y_once = mq.prefill_linear(x, qw, fused=True, keep_a=keep)
    torch.cuda.synchronize()
    assert torch.equal(_bits(y_sep), _bits(y_fus)) and torch.equal(_bits(y_sep), _bits(y_once))
    assert np.array_equal(keep.codes.cpu().numpy(), oa.codes)
    assert np.array_equal(keep.scales.cpu().numpy(), oa.scales)
    _rule_t(_out(y_sep), oracle.gemm_nvfp4_ref(oa, ow), True)


# (M, N, K) -> (W rows, A rows) per workgroup the tile choice takes on 256
# CUs for packed A, then for the fused forms (at most two A tiles): every
# reachable combination, with ragged N (a W tile group cut short) and ragged
# K among them
TILE_CASES = [
    ((128, 8192, 256), (64, 64), (64, 32)), ((128, 8232, 272), (64, 64), (64, 32)),
    ((128, 4096, 256), (32, 64), (64, 32)), ((128, 2048, 256), (32, 32), (32, 32)),
    ((100, 2056, 512), (32, 32), (32, 32)), ((32, 16384, 256), (64, 32), (64, 32)),
    ((16, 16384, 256), (64, 16), (64, 16)), ((8, 8192, 256), (32, 16), (32, 16)),
    ((5, 8200, 144), (32, 16), (32, 16)),
]


@pytest.mark.parametrize("shape,rows,fused_rows", TILE_CASES, ids=[f"{m}x{n}x{k}" for (m, n, k), _, _ in TILE_CASES])
def test_small_every_tile_choice(shape, rows, fused_rows):
    # packed, fused and quantize-once forms bit for bit, the stored A bytes,
    # and rule T on sampled output columns against the oracle
    M, N, K = shape
    announce("gemm small tiles", M, N, K, rows)
    import torch
    mq = _mq()
    xa = workloads.random_bf16((M, K), 700 + N, 1.0, "lognormal_mixed")
    xw = workloads.random_bf16((N, K), 701 + N, 0.02)
    oa = oracle.quantize_nvfp4(xa)
    qa = upload_nvfp4(oa)
    qw = mq.quantize(to_dev_bf16(xw))
    x = to_dev_bf16(xa)
    c_packed, c_fused, c_once = _c(M, N, False), _c(M, N, False), _c(M, N, False)
    mq.mq_gemm_nvfp4_prefill(qa, None, qw, c_packed, 0)
    mq.mq_gemm_nvfp4_prefill(mq.NVFP4(None, None, _rec()), x, qw, c_fused, mq.MQ_A_FUSED_BF16)
    a_once = mq.NVFP4.empty(M, K)
    mq.mq_gemm_nvfp4_prefill(a_once, x, qw, c_once, mq.MQ_A_FUSED_BF16)
    torch.cuda.synchronize()
    assert torch.equal(_bits(c_packed), _bits(c_fused)) and torch.equal(_bits(c_packed), _bits(c_once))
    assert np.array_equal(a_once.codes.cpu().numpy(), oa.codes)
    assert np.array_equal(a_once.scales.cpu().numpy(), oa.scales)
    rng = np.random.default_rng(N)
    cols = np.unique(np.concatenate([rng.choice(N, 700, replace=False), [0, N - 1]]))
    ref = oracle.gemm_nvfp4_ref(oa, oracle.quantize_nvfp4(xw, rows=cols))
    got = bf16_dev_to_f64(c_packed[:, torch.from_numpy(cols).cuda()])
    _rule_t(got, ref, True)


def test_tile_choice_as_logged():
    # MQ_LOG names each launch's workgroup rows: the cases above reach the
    # combinations they are listed with, packed and fused (a child process:
    # the flag is read once per process)
    import os
    import subprocess
    import sys
    import torch
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the expected choices are those of a 256-CU MI355X")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    shapes = [s for s, _, _ in TILE_CASES]
    script = (
        "import sys; sys.path.insert(0, {root!r})\n"
        "import torch\nimport fp4_block_scaled_elem_amd as mq\n"
        "for M, N, K in {shapes!r}:\n"
        "    x = torch.randn(M, K, device='cuda').to(torch.bfloat16)\n"
        "    qa = mq.quantize(x)\n"
        "    qw = mq.quantize(torch.randn(N, K, device='cuda').to(torch.bfloat16))\n"
        "    c = torch.empty((M, N), dtype=torch.bfloat16, device='cuda')\n"
        "    mq.mq_gemm_nvfp4_prefill(qa, None, qw, c, 0)\n"
        "    mq.prefill_linear(x, qw, out=c, fused=True)\n"
        "torch.cuda.synchronize()\nprint('done', flush=True)\n").format(root=root, shapes=shapes)
    env = dict(os.environ, MQ_LOG="1")
    r = subprocess.run([sys.executable, "-c", script], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "done" in r.stdout, r.stderr[-2000:]
    got = []
    for line in r.stderr.splitlines():
        if line.startswith("mq: gemm_small_kernel "):
            f = dict(kv.split("=") for kv in line.split()[2:] if "=" in kv)
            got.append((int(f["w_rows_per_wg"]), int(f["a_rows_per_wg"])))
    want = [r for _, packed, fused in TILE_CASES for r in (packed, fused)]
    assert got == want, got
