"""Python binding of libmq.so: NVFP4 prefill linear + BF16 decode GEMV on MI355X.

Argument marshalling only.  Every step of the path runs in the HIP kernels of
``libmq.so``; PyTorch supplies device memory and the current stream.  If the
library has not been built, every entry point raises ``LibraryNotBuilt``
(there is no fallback of any kind).

Entry points (same names as the C ABI in include/mq.h):

    mq_quantize_nvfp4(x_bf16, out: NVFP4, flags=0, stream=None)
    mq_gemm_nvfp4_prefill(a: NVFP4, a_bf16, w: NVFP4, c, flags=0, stream=None)
    mq_gemm_nvfp4_prefill_grouped(a: NVFP4, a_bf16, ws: [NVFP4], cs: [tensor], flags=0, stream=None)
    mq_gemv_bf16_decode(x_bf16, w_bf16, y_bf16, flags=0, stream=None)
    mq_gemv_bf16_decode_grouped(x_bf16, ws_bf16: [tensor], ys_bf16: [tensor], flags=0, stream=None)
    mq_gemv_nvfp4_decode(x: NVFP4, w: NVFP4, y_bf16, flags=0, stream=None)
    mq_rmsnorm_amax(x_bf16, gamma_bf16, y_bf16, rec, eps=1e-5, flags=0, stream=None)
    mq_rmsnorm_quantize_nvfp4(x_bf16, gamma_bf16, out: NVFP4, eps=1e-5, flags=0, stream=None)
    mq_swiglu_amax(a_bf16, b_bf16, y_bf16, rec, flags=0, stream=None)
    mq_linear_path / mq_linear_prepare / mq_linear_forward (through ``Linear``)

and small conveniences built on them (``quantize``, ``prefill_linear``,
``decode_linear``).
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmq.so")

# status codes and flags (mirror include/mq.h)
MQ_OK = 0
MQ_ERR_INVALID = 1
MQ_ERR_SHAPE = 2
MQ_ERR_ALIGN = 3
MQ_ERR_DEVICE = 4
MQ_ERR_LAUNCH = 5
MQ_SCALE_DYNAMIC = 0
MQ_SCALE_GIVEN = 1
MQ_OUT_BF16 = 0
MQ_OUT_F32 = 2
MQ_A_FUSED_BF16 = 4
MQ_PHASE_PREFILL = 8
MQ_PHASE_DECODE = 16
MQ_SCALE_PARTIALS = 32
MQ_PATH_DECODE_BF16 = 1
MQ_PATH_PREFILL_NVFP4 = 2
MQ_AMAX_PARTS = 1020
MQ_NOALLOC_MAX_ELEMS = 1 << 26
MQ_MAX_GROUP = 4
REC_BYTES = 16 + 4 * MQ_AMAX_PARTS  # sizeof(mq_scale_rec) = 4096

EXPORTS = ("mq_quantize_nvfp4", "mq_gemm_nvfp4_prefill", "mq_gemm_nvfp4_prefill_grouped",
           "mq_gemv_bf16_decode", "mq_gemv_bf16_decode_grouped", "mq_gemv_nvfp4_decode", "mq_rmsnorm_amax", "mq_rmsnorm_quantize_nvfp4", "mq_swiglu_amax", "mq_linear_path", "mq_linear_prepare", "mq_linear_forward",
           "mq_gemm_nvfp4_prefill_fused_noalloc", "mq_status_str", "mq_last_error", "mq_version")


class LibraryNotBuilt(ImportError):
    pass


class MQError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)}: {detail}")


class _NVFP4C(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("rec", ctypes.c_void_p)]


class _LinearC(ctypes.Structure):
    _fields_ = [("w_bf16", ctypes.c_void_p), ("w_nvfp4", _NVFP4C), ("N", ctypes.c_int64),
                ("K", ctypes.c_int64), ("prefill_min_rows", ctypes.c_int64)]


_lib = None


def lib():
    """Load libmq.so (once); raise LibraryNotBuilt if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryNotBuilt(
            f"{LIB_PATH} is missing: build it with `python -m fp4_block_scaled_elem_amd.build`")
    # torch first: its HIP runtime and the one libmq.so links against share a
    # soname, so whichever loads first serves the process; loaded first, the
    # library's copy leaves torch's device state invisible to the library
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    i64, u32, vp = ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p
    P = ctypes.POINTER(_NVFP4C)
    L.mq_quantize_nvfp4.argtypes = [vp, i64, i64, P, u32, vp]
    L.mq_quantize_nvfp4.restype = ctypes.c_int32
    L.mq_gemm_nvfp4_prefill.argtypes = [P, vp, P, vp, i64, i64, i64, u32, vp]
    L.mq_gemm_nvfp4_prefill.restype = ctypes.c_int32
    L.mq_gemm_nvfp4_prefill_grouped.argtypes = [P, vp, ctypes.c_int32, P, ctypes.POINTER(vp),
                                                ctypes.POINTER(i64), i64, i64, u32, vp]
    L.mq_gemm_nvfp4_prefill_grouped.restype = ctypes.c_int32
    L.mq_gemv_bf16_decode.argtypes = [vp, vp, vp, i64, i64, i64, u32, vp]
    L.mq_gemv_bf16_decode.restype = ctypes.c_int32
    L.mq_gemv_bf16_decode_grouped.argtypes = [vp, ctypes.c_int32, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                              ctypes.POINTER(i64), i64, i64, u32, vp]
    L.mq_gemv_bf16_decode_grouped.restype = ctypes.c_int32
    L.mq_gemv_nvfp4_decode.argtypes = [P, P, vp, i64, i64, i64, u32, vp]
    L.mq_gemv_nvfp4_decode.restype = ctypes.c_int32
    L.mq_rmsnorm_amax.argtypes = [vp, vp, vp, vp, i64, i64, ctypes.c_float, u32, vp]
    L.mq_rmsnorm_amax.restype = ctypes.c_int32
    L.mq_rmsnorm_quantize_nvfp4.argtypes = [vp, vp, i64, i64, ctypes.c_float, P, u32, vp]
    L.mq_rmsnorm_quantize_nvfp4.restype = ctypes.c_int32
    L.mq_swiglu_amax.argtypes = [vp, vp, vp, vp, i64, i64, u32, vp]
    L.mq_swiglu_amax.restype = ctypes.c_int32
    LP = ctypes.POINTER(_LinearC)
    L.mq_linear_path.argtypes = [LP, i64, u32]
    L.mq_linear_path.restype = ctypes.c_int32
    L.mq_linear_prepare.argtypes = [LP, vp]
    L.mq_linear_prepare.restype = ctypes.c_int32
    L.mq_linear_forward.argtypes = [LP, vp, i64, P, vp, u32, vp]
    L.mq_linear_forward.restype = ctypes.c_int32
    L.mq_gemm_nvfp4_prefill_fused_noalloc.argtypes = [vp, P, vp, i64, i64, i64, u32, vp]
    L.mq_gemm_nvfp4_prefill_fused_noalloc.restype = ctypes.c_int32
    L.mq_status_str.argtypes = [ctypes.c_int32]
    L.mq_status_str.restype = ctypes.c_char_p
    L.mq_last_error.argtypes = []
    L.mq_last_error.restype = ctypes.c_char_p
    L.mq_version.argtypes = []
    L.mq_version.restype = ctypes.c_char_p
    # test support (not declared in include/mq.h)
    L.mq_check_codec_steps.argtypes = [ctypes.c_int32, u32, u32, vp, u32, vp]
    L.mq_check_codec_steps.restype = ctypes.c_int32
    L.mq_check_dequant_table.argtypes = [vp, vp]
    L.mq_check_dequant_table.restype = ctypes.c_int32
    L.mq_check_mfma_rate.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp, vp]
    L.mq_check_mfma_rate.restype = ctypes.c_int32
    L.mq_check_wall_clock_khz.argtypes = [ctypes.POINTER(ctypes.c_int32)]
    L.mq_check_wall_clock_khz.restype = ctypes.c_int32
    L.mq_check_set_quant_spin_limit.argtypes = [u32]
    L.mq_check_set_quant_spin_limit.restype = u32
    L.mq_check_quant_gave_up.argtypes = []
    L.mq_check_quant_gave_up.restype = u32
    L.mq_check_set_panel_min_tiles.argtypes = [ctypes.c_int32]
    L.mq_check_set_panel_min_tiles.restype = ctypes.c_int32
    _lib = L
    return L


def status_str(s: int) -> str:
    return lib().mq_status_str(s).decode()


def last_error() -> str:
    return lib().mq_last_error().decode()


def _check(status: int, where: str):
    if status != MQ_OK:
        raise MQError(status, where, last_error())


def _stream_ptr(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev_ptr(t, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


class NVFP4:
    """Device buffers of one NVFP4 matrix [rows][cols]: packed E2M1 codes
    [rows][cols/2] (uint8), E4M3 scale bytes [rows][cols/16] (uint8) and the
    4096-byte tensor-scale record (s_t is its first binary32)."""

    def __init__(self, codes, scales, rec):
        self.codes, self.scales, self.rec = codes, scales, rec

    @classmethod
    def empty(cls, rows: int, cols: int, device="cuda"):
        import torch
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=device)
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=device)
        rec = torch.zeros(REC_BYTES // 4, dtype=torch.int32, device=device)
        return cls(codes, scales, rec)

    @property
    def shape(self):
        return (self.codes.shape[0], self.codes.shape[1] * 2)

    def s_t(self) -> float:
        """Tensor scale (synchronises)."""
        return float(self.rec[:1].view(__import__("torch").float32).item())

    def set_s_t(self, value: float):
        import torch
        self.rec[:1].view(torch.float32).fill_(value)

    def _c(self):
        return _NVFP4C(self.codes.data_ptr() if self.codes is not None else None,
                       self.scales.data_ptr() if self.scales is not None else None,
                       self.rec.data_ptr())


def mq_quantize_nvfp4(x_bf16, out: NVFP4, flags: int = MQ_SCALE_DYNAMIC, stream=None):
    import torch
    if x_bf16.dtype != torch.bfloat16 or x_bf16.dim() != 2:
        raise ValueError("x_bf16 must be a 2-D bfloat16 tensor")
    rows, cols = x_bf16.shape
    if out.shape != (rows, cols):
        raise ValueError(f"out is {out.shape}, x is {(rows, cols)}")
    oc = out._c()
    _check(lib().mq_quantize_nvfp4(_dev_ptr(x_bf16, "x_bf16"), rows, cols, ctypes.byref(oc),
                                   flags, _stream_ptr(stream)), "mq_quantize_nvfp4")


def mq_gemm_nvfp4_prefill(a: NVFP4, a_bf16, w: NVFP4, c, flags: int = 0, stream=None):
    import torch
    N, K = w.shape
    if a_bf16 is not None:
        if a_bf16.dtype != torch.bfloat16 or a_bf16.dim() != 2 or a_bf16.shape[1] != K:
            raise ValueError("a_bf16 must be bfloat16 [M][K]")
        M = a_bf16.shape[0]
    else:
        M, Ka = a.shape
        if Ka != K:
            raise ValueError(f"K mismatch: A has {Ka}, W has {K}")
    want = torch.float32 if flags & MQ_OUT_F32 else torch.bfloat16
    if c.dtype != want or tuple(c.shape) != (M, N):
        raise ValueError(f"c must be {want} [{M}][{N}]")
    ac, wc = a._c(), w._c()
    _check(lib().mq_gemm_nvfp4_prefill(ctypes.byref(ac), _dev_ptr(a_bf16, "a_bf16"), ctypes.byref(wc),
                                       _dev_ptr(c, "c"), M, N, K, flags, _stream_ptr(stream)),
           "mq_gemm_nvfp4_prefill")


def mq_gemm_nvfp4_prefill_grouped(a: NVFP4, a_bf16, ws, cs, flags: int = 0, stream=None):
    """cs[g] = A . ws[g]^T for every g, one launch (ws share K; len 1..MQ_MAX_GROUP)."""
    import torch
    if len(ws) != len(cs) or not ws:
        raise ValueError("ws and cs must be non-empty lists of the same length")
    K = ws[0].shape[1]
    if any(w.shape[1] != K for w in ws):
        raise ValueError("all weights must have the same K")
    if a_bf16 is not None:
        if a_bf16.dtype != torch.bfloat16 or a_bf16.dim() != 2 or a_bf16.shape[1] != K:
            raise ValueError("a_bf16 must be bfloat16 [M][K]")
        M = a_bf16.shape[0]
    else:
        M, Ka = a.shape
        if Ka != K:
            raise ValueError(f"K mismatch: A has {Ka}, W has {K}")
    want = torch.float32 if flags & MQ_OUT_F32 else torch.bfloat16
    for w, c in zip(ws, cs):
        if c.dtype != want or tuple(c.shape) != (M, w.shape[0]):
            raise ValueError(f"each c must be {want} [{M}][N_g]")
    n = len(ws)
    wc = (_NVFP4C * n)(*[w._c() for w in ws])
    cp = (ctypes.c_void_p * n)(*[_dev_ptr(c, "c").value for c in cs])
    nn = (ctypes.c_int64 * n)(*[w.shape[0] for w in ws])
    ac = a._c()
    _check(lib().mq_gemm_nvfp4_prefill_grouped(ctypes.byref(ac), _dev_ptr(a_bf16, "a_bf16"), n, wc, cp, nn,
                                               M, K, flags, _stream_ptr(stream)),
           "mq_gemm_nvfp4_prefill_grouped")


def mq_gemm_nvfp4_prefill_fused_noalloc(a_bf16, w: NVFP4, c, flags: int = 0, stream=None):
    """C = NVFP4(a_bf16) . W^T with the activation quantized inside the GEMM
    into the library's own scratch buffer (no caller buffers, nothing
    allocated; M * K <= MQ_NOALLOC_MAX_ELEMS).  Same output as
    mq_gemm_nvfp4_prefill with MQ_A_FUSED_BF16 and caller-owned buffers."""
    import torch
    N, K = w.shape
    if a_bf16.dtype != torch.bfloat16 or a_bf16.dim() != 2 or a_bf16.shape[1] != K:
        raise ValueError("a_bf16 must be bfloat16 [M][K]")
    M = a_bf16.shape[0]
    want = torch.float32 if flags & MQ_OUT_F32 else torch.bfloat16
    if c.dtype != want or tuple(c.shape) != (M, N):
        raise ValueError(f"c must be {want} [{M}][{N}]")
    wc = w._c()
    _check(lib().mq_gemm_nvfp4_prefill_fused_noalloc(_dev_ptr(a_bf16, "a_bf16"), ctypes.byref(wc), _dev_ptr(c, "c"),
                                                     M, N, K, flags, _stream_ptr(stream)),
           "mq_gemm_nvfp4_prefill_fused_noalloc")


def mq_gemv_bf16_decode(x_bf16, w_bf16, y_bf16, flags: int = 0, stream=None):
    import torch
    for t, n in ((x_bf16, "x"), (w_bf16, "w"), (y_bf16, "y")):
        if t.dtype != torch.bfloat16 or t.dim() != 2:
            raise ValueError(f"{n} must be a 2-D bfloat16 tensor")
    M, K = x_bf16.shape
    N = w_bf16.shape[0]
    if w_bf16.shape[1] != K or tuple(y_bf16.shape) != (M, N):
        raise ValueError("shape mismatch")
    _check(lib().mq_gemv_bf16_decode(_dev_ptr(x_bf16, "x"), _dev_ptr(w_bf16, "w"), _dev_ptr(y_bf16, "y"),
                                     M, N, K, flags, _stream_ptr(stream)), "mq_gemv_bf16_decode")


def mq_gemv_bf16_decode_grouped(x_bf16, ws_bf16, ys_bf16, flags: int = 0, stream=None):
    """ys[g] = X . ws[g]^T for every g, one launch (ws share K; len 1..MQ_MAX_GROUP)."""
    import torch
    if len(ws_bf16) != len(ys_bf16) or not ws_bf16:
        raise ValueError("ws and ys must be non-empty lists of the same length")
    if x_bf16.dtype != torch.bfloat16 or x_bf16.dim() != 2:
        raise ValueError("x must be a 2-D bfloat16 tensor")
    M, K = x_bf16.shape
    for w, y in zip(ws_bf16, ys_bf16):
        if w.dtype != torch.bfloat16 or w.dim() != 2 or w.shape[1] != K:
            raise ValueError(f"each w must be bfloat16 [N_g][{K}]")
        if y.dtype != torch.bfloat16 or tuple(y.shape) != (M, w.shape[0]):
            raise ValueError(f"each y must be bfloat16 [{M}][N_g]")
    n = len(ws_bf16)
    wp = (ctypes.c_void_p * n)(*[_dev_ptr(w, "w").value for w in ws_bf16])
    yp = (ctypes.c_void_p * n)(*[_dev_ptr(y, "y").value for y in ys_bf16])
    nn = (ctypes.c_int64 * n)(*[w.shape[0] for w in ws_bf16])
    _check(lib().mq_gemv_bf16_decode_grouped(_dev_ptr(x_bf16, "x"), n, wp, yp, nn, M, K, flags,
                                             _stream_ptr(stream)), "mq_gemv_bf16_decode_grouped")


def mq_gemv_nvfp4_decode(x: NVFP4, w: NVFP4, y_bf16, flags: int = 0, stream=None):
    """Y = X . W^T with both operands NVFP4, M <= 32 (the uniform-NVFP4 decode)."""
    import torch
    M, K = x.shape
    N, Kw = w.shape
    if Kw != K:
        raise ValueError(f"K mismatch: X has {K}, W has {Kw}")
    if y_bf16.dtype != torch.bfloat16 or tuple(y_bf16.shape) != (M, N):
        raise ValueError(f"y must be bfloat16 [{M}][{N}]")
    xc, wc = x._c(), w._c()
    _check(lib().mq_gemv_nvfp4_decode(ctypes.byref(xc), ctypes.byref(wc), _dev_ptr(y_bf16, "y"), M, N, K, flags,
                                      _stream_ptr(stream)), "mq_gemv_nvfp4_decode")


def _rec_ptr(rec):
    """An NVFP4's rec, or a rec tensor itself (REC_BYTES of device memory)."""
    t = rec.rec if isinstance(rec, NVFP4) else rec
    if t.numel() * t.element_size() != REC_BYTES:
        raise ValueError(f"rec must hold {REC_BYTES} bytes")
    return _dev_ptr(t, "rec")


def mq_rmsnorm_amax(x_bf16, gamma_bf16, y_bf16, rec, eps: float = 1e-5, flags: int = 0, stream=None):
    """y = RMSNorm(x) * gamma in bf16, and y's partial maxima into rec
    (quantize y afterwards with MQ_SCALE_PARTIALS)."""
    import torch
    if x_bf16.dtype != torch.bfloat16 or x_bf16.dim() != 2 or y_bf16.shape != x_bf16.shape \
            or y_bf16.dtype != torch.bfloat16 or gamma_bf16.dtype != torch.bfloat16 \
            or tuple(gamma_bf16.shape) != (x_bf16.shape[1],):
        raise ValueError("x, y bfloat16 [rows][cols] and gamma bfloat16 [cols]")
    rows, cols = x_bf16.shape
    _check(lib().mq_rmsnorm_amax(_dev_ptr(x_bf16, "x"), _dev_ptr(gamma_bf16, "gamma"), _dev_ptr(y_bf16, "y"),
                                 _rec_ptr(rec), rows, cols, eps, flags, _stream_ptr(stream)), "mq_rmsnorm_amax")


def mq_rmsnorm_quantize_nvfp4(x_bf16, gamma_bf16, out: NVFP4, eps: float = 1e-5, flags: int = 0, stream=None):
    """out = NVFP4(RMSNorm(x) * gamma), the bf16 RMSNorm output never
    stored (bit-identical to mq_rmsnorm_amax then MQ_SCALE_PARTIALS)."""
    import torch
    if x_bf16.dtype != torch.bfloat16 or x_bf16.dim() != 2 or gamma_bf16.dtype != torch.bfloat16 \
            or tuple(gamma_bf16.shape) != (x_bf16.shape[1],):
        raise ValueError("x bfloat16 [rows][cols] and gamma bfloat16 [cols]")
    rows, cols = x_bf16.shape
    if out.shape != (rows, cols):
        raise ValueError(f"out is {out.shape}, x is {(rows, cols)}")
    oc = out._c()
    _check(lib().mq_rmsnorm_quantize_nvfp4(_dev_ptr(x_bf16, "x"), _dev_ptr(gamma_bf16, "gamma"), rows, cols, eps,
                                           ctypes.byref(oc), flags, _stream_ptr(stream)),
           "mq_rmsnorm_quantize_nvfp4")


def mq_swiglu_amax(a_bf16, b_bf16, y_bf16, rec, flags: int = 0, stream=None):
    """y = silu(a) * b in bf16, and y's partial maxima into rec."""
    import torch
    for t, n in ((a_bf16, "a"), (b_bf16, "b"), (y_bf16, "y")):
        if t.dtype != torch.bfloat16 or t.dim() != 2 or t.shape != a_bf16.shape:
            raise ValueError(f"{n} must be bfloat16 with a's 2-D shape")
    rows, cols = a_bf16.shape
    _check(lib().mq_swiglu_amax(_dev_ptr(a_bf16, "a"), _dev_ptr(b_bf16, "b"), _dev_ptr(y_bf16, "y"),
                                _rec_ptr(rec), rows, cols, flags, _stream_ptr(stream)), "mq_swiglu_amax")


class Linear:
    """One weight W [N][K] in both formats: the original bf16 tensor (decode
    path) and its NVFP4 copy (prefill path), filled by ``prepare``.  Each
    ``forward`` goes through mq_linear_forward, which routes the call by its
    phase flag, or by its row count when it names none (M >= prefill_min_rows
    is prefill)."""

    def __init__(self, w_bf16, prefill_min_rows: int = 33):
        import torch
        if w_bf16.dtype != torch.bfloat16 or w_bf16.dim() != 2:
            raise ValueError("w_bf16 must be a 2-D bfloat16 tensor")
        self.w_bf16 = w_bf16
        self.N, self.K = w_bf16.shape
        self.w_nvfp4 = NVFP4.empty(self.N, self.K, device=w_bf16.device)
        self.prefill_min_rows = prefill_min_rows

    def _c(self):
        return _LinearC(_dev_ptr(self.w_bf16, "w_bf16").value, self.w_nvfp4._c(), self.N, self.K,
                        self.prefill_min_rows)

    def path(self, M: int, flags: int = 0) -> int:
        """MQ_PATH_DECODE_BF16, MQ_PATH_PREFILL_NVFP4, or 0 (rejected)."""
        lc = self._c()
        return lib().mq_linear_path(ctypes.byref(lc), M, flags)

    def prepare(self, stream=None):
        lc = self._c()
        _check(lib().mq_linear_prepare(ctypes.byref(lc), _stream_ptr(stream)), "mq_linear_prepare")
        return self

    def forward(self, x_bf16, out=None, flags: int = 0, a_work: NVFP4 | None = None, stream=None):
        import torch
        if x_bf16.dtype != torch.bfloat16 or x_bf16.dim() != 2 or x_bf16.shape[1] != self.K:
            raise ValueError(f"x must be bfloat16 [M][{self.K}]")
        M = x_bf16.shape[0]
        y = out if out is not None else torch.empty((M, self.N), dtype=torch.bfloat16, device=x_bf16.device)
        if y.dtype != torch.bfloat16 or tuple(y.shape) != (M, self.N):
            raise ValueError(f"out must be bfloat16 [{M}][{self.N}]")
        if a_work is None and self.path(M, flags) == MQ_PATH_PREFILL_NVFP4:
            if flags & MQ_A_FUSED_BF16:
                a_work = NVFP4(None, None, torch.zeros(REC_BYTES // 4, dtype=torch.int32, device=x_bf16.device))
            else:
                a_work = NVFP4.empty(M, self.K, device=x_bf16.device)
        lc = self._c()
        ac = a_work._c() if a_work is not None else None
        _check(lib().mq_linear_forward(ctypes.byref(lc), _dev_ptr(x_bf16, "x"), M,
                                       ctypes.byref(ac) if ac is not None else None, _dev_ptr(y, "out"),
                                       flags, _stream_ptr(stream)), "mq_linear_forward")
        return y


# ---------------------------------------------------------------- helpers --

def quantize(x_bf16, stream=None) -> NVFP4:
    q = NVFP4.empty(x_bf16.shape[0], x_bf16.shape[1], device=x_bf16.device)
    mq_quantize_nvfp4(x_bf16, q, stream=stream)
    return q


def prefill_linear(x_bf16, w: NVFP4, out=None, fused: bool = False, rec=None, keep_a: NVFP4 | None = None,
                   stream=None):
    """y = NVFP4(x) . NVFP4(W)^T in bf16, quantizing x on the fly.  fused:
    inside the GEMM launch; with keep_a (an NVFP4 of x's shape) in its
    quantize-once form, which also leaves x's NVFP4 in keep_a."""
    import torch
    M = x_bf16.shape[0]
    N = w.shape[0]
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=x_bf16.device)
    if fused:
        a = keep_a if keep_a is not None else NVFP4(None, None, rec if rec is not None else
                                                    torch.zeros(REC_BYTES // 4, dtype=torch.int32,
                                                                device=x_bf16.device))
        mq_gemm_nvfp4_prefill(a, x_bf16, w, y, MQ_A_FUSED_BF16, stream)
    else:
        a = quantize(x_bf16, stream)
        mq_gemm_nvfp4_prefill(a, None, w, y, 0, stream)
    return y


def mq_check_codec_steps(which: int, lo: int, hi: int, out, stream=None):
    """Test support: the steps of conversion `which` (0: element code, 1:
    E4M3 scale byte) over binary32 patterns lo..hi into `out` (int32 device
    tensor of 1 + 2 * cap entries; out[0] = number of steps)."""
    cap = (out.numel() - 1) // 2
    _check(lib().mq_check_codec_steps(which, lo, hi, _dev_ptr(out, "out"), cap, _stream_ptr(stream)),
           "mq_check_codec_steps")


def mq_check_dequant_table(out, stream=None):
    """Test support: binary16 operand bits of every (scale byte, code) pair
    into `out` (int16 device tensor [128][4][16])."""
    if out.numel() != 128 * 4 * 16:
        raise ValueError("out must hold 128 x 4 x 16 entries")
    _check(lib().mq_check_dequant_table(_dev_ptr(out, "out"), _stream_ptr(stream)), "mq_check_dequant_table")


def mq_check_set_quant_spin_limit(polls: int) -> int:
    """Test support: the single-launch quantizer's poll limit before a
    workgroup stops waiting for the others (0: every workgroup gives up and
    takes the maximum itself).  Returns the previous limit."""
    old = lib().mq_check_set_quant_spin_limit(polls)
    if old == 0xFFFFFFFF:
        raise MQError(MQ_ERR_DEVICE, "mq_check_set_quant_spin_limit", "HIP symbol copy failed")
    return old


def mq_check_quant_gave_up() -> int:
    """Test support: workgroups of the single-launch quantizer that gave up
    waiting since the last call (the count is reset)."""
    n = lib().mq_check_quant_gave_up()
    if n == 0xFFFFFFFF:
        raise MQError(MQ_ERR_DEVICE, "mq_check_quant_gave_up", "HIP symbol copy failed")
    return n


def mq_check_set_panel_min_tiles(tiles: int) -> int:
    """Test support: the column tiles per panel sharer from which the fused
    quantize-once GEMM takes its panel form (default 4; 1 forces it wherever
    K allows).  Returns the previous value."""
    return int(lib().mq_check_set_panel_min_tiles(tiles))


def mq_check_mfma_rate(valu_per_mfma: int, iters: int, blocks: int, sink, clocks, stream=None):
    """Measurement support: one launch of the fp16 MFMA rate kernel (0, 4 or
    6 VALU instructions per MFMA; `blocks` workgroups of four waves, each
    wave iters x 32 MFMAs of 32x32x16).  sink: float32 device tensor
    [blocks * 256]; clocks: int64 device tensor [blocks][4] (s_memtime and
    s_memrealtime at the start and the end of each block's first wave)."""
    if sink.numel() < blocks * 256 or clocks.numel() < blocks * 4:
        raise ValueError("sink or clocks too small")
    _check(lib().mq_check_mfma_rate(valu_per_mfma, iters, blocks, _dev_ptr(sink, "sink"),
                                    _dev_ptr(clocks, "clocks"), _stream_ptr(stream)), "mq_check_mfma_rate")


def wall_clock_khz() -> int:
    """Rate of the constant-rate s_memrealtime counter of the current device."""
    k = ctypes.c_int32(0)
    _check(lib().mq_check_wall_clock_khz(ctypes.byref(k)), "mq_check_wall_clock_khz")
    return int(k.value)


def decode_linear(x_bf16, w_bf16, out=None, stream=None):
    import torch
    y = out if out is not None else torch.empty((x_bf16.shape[0], w_bf16.shape[0]),
                                                dtype=torch.bfloat16, device=x_bf16.device)
    mq_gemv_bf16_decode(x_bf16, w_bf16, y, 0, stream)
    return y
