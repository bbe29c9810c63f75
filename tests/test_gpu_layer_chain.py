"""GPU parity of one 8B-shaped decoder layer's NVFP4 prefill chain.

The layer's linears as the benchmark's layer measurement runs them, at M =
4096 tokens: RMSNorm with its partial maxima -> quantization from those
partials (no amax pass) -> q and the grouped k+v GEMMs; the attention
output (a seeded stand-in: attention is torch's, not this library's) ->
two-pass quantization -> o GEMM; RMSNorm of the residual stream -> the
grouped gate+up GEMM -> SwiGLU with its partial maxima -> quantization from
those -> down GEMM.  Every link is held to the oracle on sampled rows:

* producer outputs (RMSNorm, SwiGLU) within bf16 rounding of the float64
  definitions (they are binary32 arithmetic rounded to bf16, not unique);
* every quantized activation byte for byte against ``oracle.quantize_nvfp4``
  of the bf16 tensor the GPU actually produced (whole-tensor scale);
* every GEMM output by rule T against the float64 product of the oracle's
  quantized operands;
* the RMSNorms straight to NVFP4 (as the benchmark's layer runs them now):
  the same activation bytes and tensor scales as the chain.
"""

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import announce, bf16_dev_to_f64, quantized_host, to_dev_bf16
from tests.parity import rule_t

pytestmark = pytest.mark.gpu

REL_TOL = 2.0 ** -8   # bf16 rounding (2^-9) of binary32 arithmetic, with margin
EPS = 1e-5


def _mq():
    import fp4_block_scaled_elem_amd as mq
    return mq


def _bits(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _close(y_bits, ref, what):
    y = workloads.bf16_bits_to_f32(y_bits).astype(np.float64)
    bad = np.abs(y - ref) > REL_TOL * np.abs(ref) + 1e-30
    assert not bad.any(), f"{what}: {int(bad.sum())} elements outside bf16 rounding of the oracle"


def _quant_ok(q, y_bits, rows, what):
    oq = oracle.quantize_nvfp4(y_bits, rows=rows)
    codes, scales, st = quantized_host(q)
    assert st == int(np.float32(oq.s_t).view(np.uint32)), f"{what}: tensor scale bits differ"
    assert np.array_equal(codes[rows], oq.codes), f"{what}: codes differ"
    assert np.array_equal(scales[rows], oq.scales), f"{what}: scale bytes differ"
    return oq


def _gemm_ok(c, oa, ow, rows, cols, what):
    import torch
    got = bf16_dev_to_f64(c[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()])
    r = rule_t(got, oracle.gemm_nvfp4_ref(oa, ow), bf16_out=True)
    print(f"  {what} rule T:", r, flush=True)
    assert r.ok, f"{what}: {r}"


def test_llama8b_layer_nvfp4_chain():
    announce("layer chain 8B M=4096")
    import torch
    mq = _mq()
    lay = workloads.LLAMA8B
    M, D, FF = 4096, lay.d_model, lay.d_ffn
    rng = np.random.default_rng(20261203)
    rows = np.unique(np.concatenate([rng.choice(M, 64, replace=False), [0, M - 1]]))

    def cols_of(n):
        return np.unique(np.concatenate([rng.choice(n, 128, replace=False), [0, n - 1]]))

    h = workloads.random_bf16((M, D), 501, 1.0)                 # residual stream entering the layer
    h2 = workloads.random_bf16((M, D), 502, 1.0)                # residual stream after attention (stand-in)
    xo = workloads.random_bf16((M, D), 503, 1.0)                # attention output (stand-in)
    g1 = workloads.random_bf16((D,), 504, 1.0)
    g2 = workloads.random_bf16((D,), 505, 1.0)
    wb = {p: workloads.weight(2, p) for p in workloads.PROJS}
    w = {p: mq.quantize(to_dev_bf16(b)) for p, b in wb.items()}
    out = {p: torch.empty((M, lay.proj_nk(p)[0]), dtype=torch.bfloat16, device="cuda") for p in workloads.PROJS}
    qa = {a: mq.NVFP4.empty(M, lay.act_k(a)) for a in workloads.ACTS}

    # attention block's linears
    x1 = torch.empty((M, D), dtype=torch.bfloat16, device="cuda")
    mq.mq_rmsnorm_amax(to_dev_bf16(h), to_dev_bf16(g1), x1, qa["x_qkv"], EPS)
    mq.mq_quantize_nvfp4(x1, qa["x_qkv"], mq.MQ_SCALE_PARTIALS)
    mq.mq_gemm_nvfp4_prefill(qa["x_qkv"], None, w["q"], out["q"])
    mq.mq_gemm_nvfp4_prefill_grouped(qa["x_qkv"], None, [w["k"], w["v"]], [out["k"], out["v"]])
    mq.mq_quantize_nvfp4(to_dev_bf16(xo), qa["x_o"])
    mq.mq_gemm_nvfp4_prefill(qa["x_o"], None, w["o"], out["o"])
    # MLP block's linears
    x2 = torch.empty((M, D), dtype=torch.bfloat16, device="cuda")
    mq.mq_rmsnorm_amax(to_dev_bf16(h2), to_dev_bf16(g2), x2, qa["x_gu"], EPS)
    mq.mq_quantize_nvfp4(x2, qa["x_gu"], mq.MQ_SCALE_PARTIALS)
    mq.mq_gemm_nvfp4_prefill_grouped(qa["x_gu"], None, [w["gate"], w["up"]], [out["gate"], out["up"]])
    x3 = torch.empty((M, FF), dtype=torch.bfloat16, device="cuda")
    mq.mq_swiglu_amax(out["gate"], out["up"], x3, qa["x_down"])
    mq.mq_quantize_nvfp4(x3, qa["x_down"], mq.MQ_SCALE_PARTIALS)
    mq.mq_gemm_nvfp4_prefill(qa["x_down"], None, w["down"], out["down"])
    torch.cuda.synchronize()

    ows = {}
    for p in workloads.PROJS:
        cols = cols_of(lay.proj_nk(p)[0])
        ow = oracle.quantize_nvfp4(wb[p], rows=cols)
        codes, scales, st = quantized_host(w[p])
        assert st == int(np.float32(ow.s_t).view(np.uint32)) and np.array_equal(codes[cols], ow.codes) \
            and np.array_equal(scales[cols], ow.scales), f"weight {p} differs from the oracle"
        ows[p] = (ow, cols)

    # the producers
    x1b, x2b, x3b = _bits(x1), _bits(x2), _bits(x3)
    _close(x1b[rows], oracle.rmsnorm_ref(h[rows], g1, EPS), "RMSNorm (attention input)")
    _close(x2b[rows], oracle.rmsnorm_ref(h2[rows], g2, EPS), "RMSNorm (MLP input)")
    gate_b, up_b = _bits(out["gate"]), _bits(out["up"])
    _close(x3b[rows], oracle.swiglu_ref(gate_b[rows], up_b[rows]), "SwiGLU")

    # quantized activations (whole-tensor scale from what the GPU produced)
    oa = {"x_qkv": _quant_ok(qa["x_qkv"], x1b, rows, "x_qkv from RMSNorm partials"),
          "x_o": _quant_ok(qa["x_o"], xo, rows, "x_o"),
          "x_gu": _quant_ok(qa["x_gu"], x2b, rows, "x_gu from RMSNorm partials"),
          "x_down": _quant_ok(qa["x_down"], x3b, rows, "x_down from SwiGLU partials")}

    # every projection's output
    for p in workloads.PROJS:
        ow, cols = ows[p]
        _gemm_ok(out[p], oa[workloads.PROJ_INPUT[p]], ow, rows, cols, p)

    # the RMSNorms straight to NVFP4 (their bf16 outputs never stored): the
    # same activation bytes and tensor scales as the chain above
    for a, hb, gb in (("x_qkv", h, g1), ("x_gu", h2, g2)):
        qf = mq.NVFP4.empty(M, D)
        mq.mq_rmsnorm_quantize_nvfp4(to_dev_bf16(hb), to_dev_bf16(gb), qf, EPS)
        torch.cuda.synchronize()
        assert torch.equal(qf.codes, qa[a].codes) and torch.equal(qf.scales, qa[a].scales), a
        assert torch.equal(qf.rec[:1], qa[a].rec[:1]), f"{a}: tensor scale"
