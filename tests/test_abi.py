"""The C ABI: libmq.so loads, exports every function include/mq.h declares,
and rejects bad arguments with the documented status before any HIP call
(CPU; no kernel is launched)."""

import ctypes
import os
import re

import pytest

import fp4_block_scaled_elem_amd as mq

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mq.h")


def _header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mq_[a-z0-9_]+)\s*\(", src)))


def _header_defines():
    out = {}
    for m in re.finditer(r"#define\s+(MQ_[A-Z0-9_]+)\s+(\d+)u?", open(HEADER).read()):
        out[m.group(1)] = int(m.group(2))
    return out


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mq.LIB_PATH):
        pytest.skip("libmq.so not built")
    return mq.lib()


def test_header_declares_the_entry_points():
    fns = _header_functions()
    for f in ("mq_quantize_nvfp4", "mq_gemm_nvfp4_prefill", "mq_gemm_nvfp4_prefill_grouped",
              "mq_gemv_bf16_decode", "mq_gemv_nvfp4_decode", "mq_rmsnorm_amax", "mq_swiglu_amax",
              "mq_rmsnorm_quantize_nvfp4",
              "mq_linear_path", "mq_linear_prepare", "mq_linear_forward"):
        assert f in fns


def test_every_declared_symbol_is_exported(L):
    for f in _header_functions():
        assert hasattr(L, f), f
    assert set(_header_functions()) <= set(mq.EXPORTS)


def test_python_constants_match_header():
    d = _header_defines()
    for k, v in d.items():
        assert getattr(mq, k) == v, k
    assert mq.REC_BYTES == 4096


def test_status_strings(L):
    for code, name in [(0, "MQ_OK"), (1, "MQ_ERR_INVALID"), (2, "MQ_ERR_SHAPE"), (3, "MQ_ERR_ALIGN"),
                       (4, "MQ_ERR_DEVICE"), (5, "MQ_ERR_LAUNCH")]:
        assert mq.status_str(code) == name
    assert L.mq_version().decode().startswith("mq ")


# fake, never dereferenced device addresses (checks happen first)
P16 = 0x10000
P8 = 0x10008
P1 = 0x10001


def _q(codes, scales, rec):
    return ctypes.byref(mq._NVFP4C(codes, scales, rec))


def test_quantize_argument_errors(L):
    f = L.mq_quantize_nvfp4
    assert f(None, 4, 16, _q(P16, P16, P16), 0, None) == mq.MQ_ERR_INVALID
    assert f(P16, 4, 16, None, 0, None) == mq.MQ_ERR_INVALID
    assert f(P16, 4, 16, _q(None, P16, P16), 0, None) == mq.MQ_ERR_INVALID
    assert f(P16, 4, 16, _q(P16, P16, P16), 8, None) == mq.MQ_ERR_INVALID
    assert "flags" in mq.last_error()
    assert f(P16, 0, 16, _q(P16, P16, P16), 0, None) == mq.MQ_ERR_SHAPE
    assert f(P16, 4, 24, _q(P16, P16, P16), 0, None) == mq.MQ_ERR_SHAPE
    assert f(P16, 4, -16, _q(P16, P16, P16), 0, None) == mq.MQ_ERR_SHAPE
    assert f(P16, 1 << 31, 16, _q(P16, P16, P16), 0, None) == mq.MQ_ERR_SHAPE
    assert f(P8, 4, 16, _q(P16, P16, P16), 0, None) == mq.MQ_ERR_ALIGN
    assert f(P16, 4, 16, _q(P8, P16, P16), 0, None) == mq.MQ_ERR_ALIGN
    assert f(P16, 4, 16, _q(P16, P1, P16), 0, None) == mq.MQ_ERR_ALIGN
    assert f(P16, 4, 16, _q(P16, P16, P8), 0, None) == mq.MQ_ERR_ALIGN


def test_gemm_argument_errors(L):
    f = L.mq_gemm_nvfp4_prefill
    a, w = _q(P16, P16, P16), _q(P16, P16, P16)
    assert f(None, None, w, P16, 4, 4, 16, 0, None) == mq.MQ_ERR_INVALID
    assert f(a, None, None, P16, 4, 4, 16, 0, None) == mq.MQ_ERR_INVALID
    assert f(a, None, w, None, 4, 4, 16, 0, None) == mq.MQ_ERR_INVALID
    assert f(a, None, w, P16, 4, 4, 16, 64, None) == mq.MQ_ERR_INVALID
    assert f(a, None, w, P16, 4, 4, 16, mq.MQ_SCALE_GIVEN, None) == mq.MQ_ERR_INVALID
    assert f(a, P16, w, P16, 4, 4, 16, 0, None) == mq.MQ_ERR_INVALID             # a_bf16 without fused
    assert f(a, None, w, P16, 4, 4, 16, mq.MQ_A_FUSED_BF16, None) == mq.MQ_ERR_INVALID
    assert f(_q(None, None, P16), None, w, P16, 4, 4, 16, 0, None) == mq.MQ_ERR_INVALID
    assert f(a, None, w, P16, 4, 4, 40, 0, None) == mq.MQ_ERR_SHAPE
    assert f(a, None, w, P16, 0, 4, 16, 0, None) == mq.MQ_ERR_SHAPE
    assert f(a, None, w, P16, 4, 0, 16, 0, None) == mq.MQ_ERR_SHAPE
    assert f(a, None, w, P16, 4, 4, 0, 0, None) == mq.MQ_ERR_SHAPE
    assert f(a, None, w, P8, 4, 4, 16, 0, None) == mq.MQ_ERR_ALIGN
    assert f(_q(P8, P16, P16), None, w, P16, 4, 4, 16, 0, None) == mq.MQ_ERR_ALIGN
    assert f(a, None, _q(P16, P1, P16), P16, 4, 4, 16, 0, None) == mq.MQ_ERR_ALIGN
    assert f(_q(None, None, P16), P8, w, P16, 4, 4, 16, mq.MQ_A_FUSED_BF16, None) == mq.MQ_ERR_ALIGN
    # fused with A's buffers (the quantize-once form): both or neither, aligned
    fz = mq.MQ_A_FUSED_BF16
    assert f(_q(P16, None, P16), P16, w, P16, 4, 4, 16, fz, None) == mq.MQ_ERR_INVALID
    assert f(_q(None, P16, P16), P16, w, P16, 4, 4, 16, fz, None) == mq.MQ_ERR_INVALID
    assert f(_q(P8, P16, P16), P16, w, P16, 4, 4, 16, fz, None) == mq.MQ_ERR_ALIGN
    assert f(_q(P16, P1, P16), P16, w, P16, 4, 4, 16, fz, None) == mq.MQ_ERR_ALIGN


def _grouped(L, a, a_bf16, ws, cs, ns, M=4, K=16, flags=0, n_group=None):
    n = len(ws)
    wa = (mq._NVFP4C * max(n, 1))(*[mq._NVFP4C(*w) for w in ws])
    ca = (ctypes.c_void_p * max(n, 1))(*cs)
    na = (ctypes.c_int64 * max(n, 1))(*ns)
    return L.mq_gemm_nvfp4_prefill_grouped(a, a_bf16, n if n_group is None else n_group, wa, ca, na, M, K,
                                           flags, None)


def test_grouped_gemm_argument_errors(L):
    a = _q(P16, P16, P16)
    w = (P16, P16, P16)
    g = lambda **kw: _grouped(L, a, None, [w, w], [P16, P16], [4, 4], **kw)
    assert g(n_group=0) == mq.MQ_ERR_INVALID
    assert g(n_group=mq.MQ_MAX_GROUP + 1) == mq.MQ_ERR_INVALID
    assert "n_group" in mq.last_error()
    assert g(flags=64) == mq.MQ_ERR_INVALID
    assert L.mq_gemm_nvfp4_prefill_grouped(a, None, 1, None, None, None, 4, 16, 0, None) == mq.MQ_ERR_INVALID
    assert _grouped(L, a, None, [w, (P16, None, P16)], [P16, P16], [4, 4]) == mq.MQ_ERR_INVALID
    assert _grouped(L, a, None, [w, w], [P16, None], [4, 4]) == mq.MQ_ERR_INVALID
    assert "group 1" in mq.last_error()
    assert _grouped(L, a, None, [w, w], [P16, P16], [4, 0]) == mq.MQ_ERR_SHAPE
    assert g(K=40) == mq.MQ_ERR_SHAPE
    assert _grouped(L, a, None, [w, w], [P16, P16], [1 << 30, 1 << 30], M=1) == mq.MQ_ERR_SHAPE
    assert _grouped(L, a, None, [w, w], [P16, P8], [4, 4]) == mq.MQ_ERR_ALIGN
    assert _grouped(L, a, None, [w, (P16, P1, P16)], [P16, P16], [4, 4]) == mq.MQ_ERR_ALIGN
    assert _grouped(L, _q(None, None, P16), P8, [w], [P16], [4], flags=mq.MQ_A_FUSED_BF16) == mq.MQ_ERR_ALIGN


def test_gemv_argument_errors(L):
    f = L.mq_gemv_bf16_decode
    assert f(None, P16, P16, 1, 4, 16, 0, None) == mq.MQ_ERR_INVALID
    assert f(P16, P16, P16, 1, 4, 16, 1, None) == mq.MQ_ERR_INVALID
    assert f(P16, P16, P16, 0, 4, 16, 0, None) == mq.MQ_ERR_SHAPE
    assert f(P16, P16, P16, 33, 4, 16, 0, None) == mq.MQ_ERR_SHAPE
    assert f(P16, P16, P16, 1, 4, 17, 0, None) == mq.MQ_ERR_SHAPE
    assert f(P16, P16, P16, 1, 0, 16, 0, None) == mq.MQ_ERR_SHAPE
    assert f(P8, P16, P16, 1, 4, 16, 0, None) == mq.MQ_ERR_ALIGN
    assert f(P16, P16, P1, 1, 4, 16, 0, None) == mq.MQ_ERR_ALIGN


def test_grouped_gemv_argument_errors(L):
    f = L.mq_gemv_bf16_decode_grouped

    def call(x, ws, ys, ns, M=1, K=16, flags=0, n_group=None):
        n = len(ws) if n_group is None else n_group
        m = max(len(ws), 1)
        wa = (ctypes.c_void_p * m)(*(ws or [None]))
        ya = (ctypes.c_void_p * m)(*(ys or [None]))
        na = (ctypes.c_int64 * m)(*(ns or [1]))
        return f(x, n, wa, ya, na, M, K, flags, None)

    assert call(P16, [P16], [P16], [4], flags=1) == mq.MQ_ERR_INVALID
    assert call(P16, [P16], [P16], [4], n_group=0) == mq.MQ_ERR_INVALID
    assert call(P16, [P16] * 5, [P16] * 5, [4] * 5) == mq.MQ_ERR_INVALID    # more than MQ_MAX_GROUP
    assert call(None, [P16], [P16], [4]) == mq.MQ_ERR_INVALID
    assert call(P16, [P16, None], [P16, P16], [4, 4]) == mq.MQ_ERR_INVALID
    assert call(P16, [P16, P16], [P16, None], [4, 4]) == mq.MQ_ERR_INVALID
    assert f(P16, 1, None, None, None, 1, 16, 0, None) == mq.MQ_ERR_INVALID
    assert call(P16, [P16], [P16], [4], M=0) == mq.MQ_ERR_SHAPE
    assert call(P16, [P16], [P16], [4], M=33) == mq.MQ_ERR_SHAPE
    assert call(P16, [P16], [P16], [4], K=24) == mq.MQ_ERR_SHAPE
    assert call(P16, [P16, P16], [P16, P16], [4, 0]) == mq.MQ_ERR_SHAPE
    assert call(P8, [P16], [P16], [4]) == mq.MQ_ERR_ALIGN
    assert call(P16, [P16, P8], [P16, P16], [4, 4]) == mq.MQ_ERR_ALIGN
    assert call(P16, [P16], [P1], [4]) == mq.MQ_ERR_ALIGN


def test_gemv_nvfp4_argument_errors(L):
    f = L.mq_gemv_nvfp4_decode
    q = _q(P16, P16, P16)
    assert f(None, q, P16, 1, 4, 16, 0, None) == mq.MQ_ERR_INVALID
    assert f(q, None, P16, 1, 4, 16, 0, None) == mq.MQ_ERR_INVALID
    assert f(q, q, None, 1, 4, 16, 0, None) == mq.MQ_ERR_INVALID
    assert f(q, _q(P16, None, P16), P16, 1, 4, 16, 0, None) == mq.MQ_ERR_INVALID
    assert f(q, q, P16, 1, 4, 16, 1, None) == mq.MQ_ERR_INVALID
    assert f(q, q, P16, 0, 4, 16, 0, None) == mq.MQ_ERR_SHAPE
    assert f(q, q, P16, 33, 4, 16, 0, None) == mq.MQ_ERR_SHAPE
    assert f(q, q, P16, 1, 4, 24, 0, None) == mq.MQ_ERR_SHAPE
    assert f(q, q, P16, 1, 0, 16, 0, None) == mq.MQ_ERR_SHAPE
    assert f(_q(P8, P16, P16), q, P16, 1, 4, 16, 0, None) == mq.MQ_ERR_ALIGN
    assert f(q, _q(P16, P1, P16), P16, 1, 4, 16, 0, None) == mq.MQ_ERR_ALIGN
    assert f(q, _q(P16, P16, P8), P16, 1, 4, 16, 0, None) == mq.MQ_ERR_ALIGN
    assert f(q, q, P1, 1, 4, 16, 0, None) == mq.MQ_ERR_ALIGN


def test_producer_argument_errors(L):
    r = L.mq_rmsnorm_amax
    assert r(None, P16, P16 + 16, P16, 4, 16, 1e-5, 0, None) == mq.MQ_ERR_INVALID
    assert r(P16, P16, P16 + 16, None, 4, 16, 1e-5, 0, None) == mq.MQ_ERR_INVALID
    assert r(P16, P16, P16 + 16, P16, 4, 16, 1e-5, 1, None) == mq.MQ_ERR_INVALID
    assert r(P16, P16, P16 + 16, P16, 4, 16, -1.0, 0, None) == mq.MQ_ERR_INVALID
    assert r(P16, P16, P16 + 16, P16, 4, 16, float("nan"), 0, None) == mq.MQ_ERR_INVALID
    assert r(P16, P16, P16, P16, 4, 16, 1e-5, 0, None) == mq.MQ_ERR_INVALID              # y aliases x
    assert r(P16, P16, P16 + 16, P16, 0, 16, 1e-5, 0, None) == mq.MQ_ERR_SHAPE
    assert r(P16, P16, P16 + 16, P16, 4, 24, 1e-5, 0, None) == mq.MQ_ERR_SHAPE
    assert r(P8, P16, P16 + 16, P16, 4, 16, 1e-5, 0, None) == mq.MQ_ERR_ALIGN
    assert r(P16, P16, P16 + 16, P8, 4, 16, 1e-5, 0, None) == mq.MQ_ERR_ALIGN
    rq = L.mq_rmsnorm_quantize_nvfp4
    assert rq(None, P16, 4, 16, 1e-5, _q(P16, P16, P16), 0, None) == mq.MQ_ERR_INVALID
    assert rq(P16, P16, 4, 16, 1e-5, None, 0, None) == mq.MQ_ERR_INVALID
    assert rq(P16, P16, 4, 16, 1e-5, _q(P16, None, P16), 0, None) == mq.MQ_ERR_INVALID
    assert rq(P16, P16, 4, 16, 1e-5, _q(P16, P16, P16), 1, None) == mq.MQ_ERR_INVALID
    assert rq(P16, P16, 4, 16, -1.0, _q(P16, P16, P16), 0, None) == mq.MQ_ERR_INVALID
    assert rq(P16, P16, 0, 16, 1e-5, _q(P16, P16, P16), 0, None) == mq.MQ_ERR_SHAPE
    assert rq(P16, P16, 4, 24, 1e-5, _q(P16, P16, P16), 0, None) == mq.MQ_ERR_SHAPE
    assert rq(P8, P16, 4, 16, 1e-5, _q(P16, P16, P16), 0, None) == mq.MQ_ERR_ALIGN
    assert rq(P16, P16, 4, 16, 1e-5, _q(P8, P16, P16), 0, None) == mq.MQ_ERR_ALIGN
    assert rq(P16, P16, 4, 16, 1e-5, _q(P16, P1, P16), 0, None) == mq.MQ_ERR_ALIGN
    s = L.mq_swiglu_amax
    assert s(P16, None, P16 + 16, P16, 4, 16, 0, None) == mq.MQ_ERR_INVALID
    assert s(P16, P16, P16 + 16, P16, 4, 16, 2, None) == mq.MQ_ERR_INVALID
    assert s(P16, P16 + 16, P16 + 16, P16, 4, 16, 0, None) == mq.MQ_ERR_INVALID          # y aliases b
    assert s(P16, P16, P16 + 16, P16, 4, 0, 0, None) == mq.MQ_ERR_SHAPE
    assert s(P16, P16, P8, P16, 4, 16, 0, None) == mq.MQ_ERR_ALIGN
    # the partial-maxima flag: exclusive with a given scale, GEMM only with the fused prologue
    q = L.mq_quantize_nvfp4
    assert q(P16, 4, 16, _q(P16, P16, P16), mq.MQ_SCALE_GIVEN | mq.MQ_SCALE_PARTIALS, None) == mq.MQ_ERR_INVALID
    g = L.mq_gemm_nvfp4_prefill
    assert g(_q(P16, P16, P16), None, _q(P16, P16, P16), P16, 4, 4, 16, mq.MQ_SCALE_PARTIALS,
             None) == mq.MQ_ERR_INVALID


def _lin(w=P16, codes=P16, scales=P16, rec=P16, N=4, K=16, pmin=33):
    return ctypes.byref(mq._LinearC(w, mq._NVFP4C(codes, scales, rec), N, K, pmin))


def test_linear_path_routing(L):
    # the phase flag decides; without one the row count does (M >= pmin is
    # prefill); a decode call takes at most 32 rows
    f = L.mq_linear_path
    D, P = mq.MQ_PATH_DECODE_BF16, mq.MQ_PATH_PREFILL_NVFP4
    for M in (1, 2, 16, 31, 32):
        assert f(_lin(), M, 0) == D
    for M in (33, 64, 4096, 1 << 20):
        assert f(_lin(), M, 0) == P
    assert f(_lin(pmin=1), 1, 0) == P
    assert f(_lin(pmin=17), 16, 0) == D and f(_lin(pmin=17), 17, 0) == P
    assert f(_lin(), 1, mq.MQ_PHASE_PREFILL) == P
    assert f(_lin(), 4096, mq.MQ_PHASE_PREFILL | mq.MQ_A_FUSED_BF16) == P
    assert f(_lin(), 32, mq.MQ_PHASE_DECODE) == D
    assert f(_lin(pmin=1), 5, mq.MQ_PHASE_DECODE) == D
    assert f(_lin(), 33, mq.MQ_PHASE_DECODE) == 0
    assert f(_lin(), 1, mq.MQ_PHASE_PREFILL | mq.MQ_PHASE_DECODE) == 0
    assert f(_lin(), 0, 0) == 0
    assert f(_lin(pmin=0), 1, 0) == 0 and f(_lin(pmin=34), 1, 0) == 0
    assert f(None, 1, 0) == 0


def test_linear_argument_errors(L):
    fw, fp = L.mq_linear_forward, L.mq_linear_prepare
    a = _q(P16, P16, P16)
    assert fp(None, None) == mq.MQ_ERR_INVALID
    assert fp(_lin(w=None), None) == mq.MQ_ERR_INVALID
    assert fp(_lin(rec=None), None) == mq.MQ_ERR_INVALID
    assert fp(_lin(K=24), None) == mq.MQ_ERR_SHAPE
    assert fp(_lin(N=0), None) == mq.MQ_ERR_SHAPE
    assert fp(_lin(w=P8), None) == mq.MQ_ERR_ALIGN
    assert fp(_lin(scales=P1), None) == mq.MQ_ERR_ALIGN
    assert fw(_lin(), P16, 1, None, P16, 64, None) == mq.MQ_ERR_INVALID                   # unknown flag
    assert fw(_lin(), P16, 1, None, P16, mq.MQ_PHASE_PREFILL | mq.MQ_PHASE_DECODE, None) == mq.MQ_ERR_INVALID
    assert fw(None, P16, 1, None, P16, 0, None) == mq.MQ_ERR_INVALID
    assert fw(_lin(pmin=34), P16, 1, None, P16, 0, None) == mq.MQ_ERR_INVALID
    assert fw(_lin(), None, 1, None, P16, 0, None) == mq.MQ_ERR_INVALID
    assert fw(_lin(), P16, 1, None, None, 0, None) == mq.MQ_ERR_INVALID
    assert fw(_lin(), P16, 0, None, P16, 0, None) == mq.MQ_ERR_SHAPE
    assert fw(_lin(), P16, 40, a, P16, mq.MQ_PHASE_DECODE, None) == mq.MQ_ERR_SHAPE
    assert "decode" in mq.last_error()
    assert fw(_lin(), P8, 1, None, P16, 0, None) == mq.MQ_ERR_ALIGN
    assert fw(_lin(), P16, 1, None, P1, 0, None) == mq.MQ_ERR_ALIGN                        # decode: y 2-byte
    # prefill calls need a_work (its rec always; codes and scales unless fused)
    assert fw(_lin(), P16, 64, None, P16, 0, None) == mq.MQ_ERR_INVALID
    assert fw(_lin(), P16, 64, _q(P16, P16, None), P16, 0, None) == mq.MQ_ERR_INVALID
    assert fw(_lin(), P16, 64, _q(None, P16, P16), P16, 0, None) == mq.MQ_ERR_INVALID
    assert fw(_lin(), P16, 64, _q(P16, P1, P16), P16, 0, None) == mq.MQ_ERR_ALIGN
    assert fw(_lin(), P16, 64, a, P8, 0, None) == mq.MQ_ERR_ALIGN                          # prefill: y 16-byte
    assert fw(_lin(), P16, 1, a, P8, mq.MQ_PHASE_PREFILL, None) == mq.MQ_ERR_ALIGN
    assert fw(_lin(N=1 << 30), P16, 1 << 11, a, P16, 0, None) == mq.MQ_ERR_SHAPE


def _no_gpu():
    try:
        import torch
        return torch.cuda.device_count() == 0
    except Exception:
        return True


@pytest.mark.skipif(not _no_gpu(), reason="valid fake pointers would be launched on a real GPU")
def test_noalloc_gemm_argument_errors(L):
    f = L.mq_gemm_nvfp4_prefill_fused_noalloc
    w = _q(P16, P16, P16)
    assert f(None, w, P16, 4, 16, 16, 0, None) == mq.MQ_ERR_INVALID
    assert f(P16, None, P16, 4, 16, 16, 0, None) == mq.MQ_ERR_INVALID
    assert f(P16, w, None, 4, 16, 16, 0, None) == mq.MQ_ERR_INVALID
    for flags in (mq.MQ_SCALE_GIVEN, mq.MQ_SCALE_PARTIALS, 64):
        assert f(P16, w, P16, 4, 16, 16, flags, None) == mq.MQ_ERR_INVALID
    assert f(P16, w, P16, 0, 16, 16, 0, None) == mq.MQ_ERR_SHAPE
    assert f(P16, w, P16, 4, 16, 24, 0, None) == mq.MQ_ERR_SHAPE
    # one row past the scratch buffer's capacity
    assert f(P16, w, P16, mq.MQ_NOALLOC_MAX_ELEMS // 4096 + 1, 16, 4096, 0, None) == mq.MQ_ERR_SHAPE
    assert "scratch" in mq.last_error()


def test_valid_arguments_without_a_gpu_report_device_error(L):
    assert L.mq_quantize_nvfp4(P16, 4, 16, _q(P16, P16, P16), 0, None) == mq.MQ_ERR_DEVICE
    assert L.mq_gemm_nvfp4_prefill(_q(P16, P16, P16), None, _q(P16, P16, P16), P16, 4, 4, 16, 0,
                                   None) == mq.MQ_ERR_DEVICE
    assert L.mq_gemv_bf16_decode(P16, P16, P16, 1, 4, 16, 0, None) == mq.MQ_ERR_DEVICE
    wa, ya, na = (ctypes.c_void_p * 2)(P16, P16), (ctypes.c_void_p * 2)(P16, P16), (ctypes.c_int64 * 2)(4, 8)
    assert L.mq_gemv_bf16_decode_grouped(P16, 2, wa, ya, na, 1, 16, 0, None) == mq.MQ_ERR_DEVICE
    assert L.mq_gemm_nvfp4_prefill(_q(P16, P16, P16), P16, _q(P16, P16, P16), P16, 4, 4, 16,
                                   mq.MQ_A_FUSED_BF16, None) == mq.MQ_ERR_DEVICE
    w = (P16, P16, P16)
    assert _grouped(L, _q(P16, P16, P16), None, [w, w, w], [P16, P16, P16], [4, 8, 12]) == mq.MQ_ERR_DEVICE
    assert L.mq_gemv_nvfp4_decode(_q(P16, P16, P16), _q(P16, P16, P16), P16, 1, 4, 16, 0,
                                  None) == mq.MQ_ERR_DEVICE
    assert L.mq_rmsnorm_amax(P16, P16, P16 + 16, P16, 4, 16, 1e-5, 0, None) == mq.MQ_ERR_DEVICE
    assert L.mq_swiglu_amax(P16, P16 + 16, P16 + 32, P16, 4, 16, 0, None) == mq.MQ_ERR_DEVICE
    assert L.mq_rmsnorm_quantize_nvfp4(P16, P16, 4, 16, 1e-5, _q(P16, P16, P16), 0, None) == mq.MQ_ERR_DEVICE
    assert L.mq_quantize_nvfp4(P16, 4, 16, _q(P16, P16, P16), mq.MQ_SCALE_PARTIALS, None) == mq.MQ_ERR_DEVICE
    assert L.mq_linear_prepare(_lin(), None) == mq.MQ_ERR_DEVICE
    assert L.mq_linear_forward(_lin(), P16, 1, None, P1 + 1, 0, None) == mq.MQ_ERR_DEVICE
    assert L.mq_linear_forward(_lin(), P16, 64, _q(P16, P16, P16), P16, 0, None) == mq.MQ_ERR_DEVICE
    assert L.mq_linear_forward(_lin(), P16, 64, _q(None, None, P16), P16, mq.MQ_A_FUSED_BF16,
                               None) == mq.MQ_ERR_DEVICE
    assert mq.last_error()


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(mq, "_lib", None)
    monkeypatch.setattr(mq, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(mq.LibraryNotBuilt):
        mq.lib()
