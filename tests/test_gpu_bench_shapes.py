"""GPU parity of every launch the benchmark times, at the configurations' full shapes.

The benchmark's step is one pass over a decoder layer's seven projections,
launched as q, k+v, o, gate+up and down (k with v and gate with up share one
launch each, since they read the same activation).  Each test below runs one
such launch exactly as the benchmark does, on the same seeded inputs, and
holds it to the oracle:

* the NVFP4 weights: codes and scale bytes of sampled rows and the tensor
  scale bits, byte for byte against ``oracle.quantize_nvfp4``;
* A's NVFP4 (written by the standalone quantizer, or by the GEMM itself in
  the fused prologue's quantize-once form): bit-identical to the standalone
  quantizer over the whole tensor, and byte for byte against the oracle on
  sampled rows (with the tensor scale of the whole input);
* the bf16 output: rule T against the float64 oracle on sampled rows x
  sampled columns of every group, and (fused forms) bit-identical over the
  whole output to quantize-then-GEMM.

Long-context configuration: M = 32768 tokens of Student-t activations, the
quantization fused into every GEMM (quantize-once form: each workgroup
quantizes the 256-row panel of A it reads, once, into A's NVFP4 buffers;
the per-tile form, which re-quantizes A for every column tile, for q and
gate).  70B-shaped slice: M = 16384, K = 8192 / 28672, separate quantizer
then GEMM.  8B prefill: the grouped k+v launch (256x128 tiles) the other
GEMM tests cover only as single calls.
"""

import functools

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import announce, bf16_dev_to_f64, quantized_host, to_dev_bf16
from tests.parity import rule_t

pytestmark = pytest.mark.gpu

LAUNCHES = (("q",), ("k", "v"), ("o",), ("gate", "up"), ("down",))


def _mq():
    import fp4_block_scaled_elem_amd as mq
    return mq


@functools.lru_cache(maxsize=2)
def _act_host(cfg, act):
    return workloads.activation(cfg, act)


@functools.lru_cache(maxsize=1)
def _act_dev(cfg, act):
    return to_dev_bf16(_act_host(cfg, act))


def _release():
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _sample(n, k, seed, edges=()):
    rng = np.random.default_rng(seed)
    pick = rng.choice(n, min(k, n), replace=False)
    return np.unique(np.concatenate([pick, [e for e in edges if e < n]]).astype(np.int64))


def _same(a, b):
    import torch
    v = torch.int32 if a.dtype == torch.float32 else torch.int16
    return torch.equal(a.view(v), b.view(v))


def _check_weight(mq, cfg, proj, cols):
    """GPU-quantized weight of `proj`; its sampled rows against the oracle."""
    xw = workloads.weight(cfg, proj)
    qw = mq.quantize(to_dev_bf16(xw))
    ow = oracle.quantize_nvfp4(xw, rows=cols)
    codes, scales, st = quantized_host(qw)
    assert st == int(np.float32(ow.s_t).view(np.uint32)), f"{proj}: weight tensor scale bits differ"
    assert np.array_equal(codes[cols], ow.codes), f"{proj}: weight codes differ from the oracle"
    assert np.array_equal(scales[cols], ow.scales), f"{proj}: weight scale bytes differ from the oracle"
    return qw, ow


def _check_a_bytes(q, xa, rows, what):
    """A's NVFP4 on the device against the oracle on sampled rows."""
    oa = oracle.quantize_nvfp4(xa, rows=rows)
    codes, scales, st = quantized_host(q)
    assert st == int(np.float32(oa.s_t).view(np.uint32)), f"{what}: A's tensor scale bits differ"
    assert np.array_equal(codes[rows], oa.codes), f"{what}: A's codes differ from the oracle"
    assert np.array_equal(scales[rows], oa.scales), f"{what}: A's scale bytes differ from the oracle"
    return oa


def _check_output(c, oa, ow, rows, cols, what):
    import torch
    ref = oracle.gemm_nvfp4_ref(oa, ow)
    got = bf16_dev_to_f64(c[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()])
    r = rule_t(got, ref, bf16_out=True)
    print(f"  {what} rule T:", r, flush=True)
    assert r.ok, f"{what}: {r}"


def _launch(mq, a, x, qws, cs, flags):
    import torch
    if len(qws) == 1:
        mq.mq_gemm_nvfp4_prefill(a, x, qws[0], cs[0], flags)
    else:
        mq.mq_gemm_nvfp4_prefill_grouped(a, x, qws, cs, flags)
    torch.cuda.synchronize()


def _run_launch(cfg, projs, form):
    """One benchmark launch of configuration `cfg` over `projs`.

    form: "separate" (standalone quantizer, then the GEMM), "panel" (fused,
    quantize-once) or "tile" (fused, per-tile re-quantization)."""
    import torch
    mq = _mq()
    act = workloads.PROJ_INPUT[projs[0]]
    xa = _act_host(cfg, act)
    x = _act_dev(cfg, act)
    M, K = xa.shape
    seed = 1000 * cfg + 10 * len(projs) + workloads.PROJS.index(projs[0])
    rows = _sample(M, 96, seed, edges=(0, 255, 256, M - 256, M - 1))
    qws, ows, colss = [], [], []
    for i, p in enumerate(projs):
        N = workloads.CONFIGS[cfg].layer.proj_nk(p)[0]
        cols = _sample(N, 160, seed + 1 + i, edges=(0, 127, 128, 255, 256, N - 1))
        qw, ow = _check_weight(mq, cfg, p, cols)
        qws.append(qw)
        ows.append(ow)
        colss.append(cols)
    cs = [torch.empty((M, qw.shape[0]), dtype=torch.bfloat16, device="cuda") for qw in qws]
    qa = mq.quantize(x)  # the standalone quantizer (the separate path's A)
    if form == "separate":
        _launch(mq, qa, None, qws, cs, 0)
        oa = _check_a_bytes(qa, xa, rows, f"cfg{cfg} {projs}")
    else:
        if form == "panel":
            a = mq.NVFP4.empty(M, K)
        else:
            a = mq.NVFP4(None, None, torch.zeros(mq.REC_BYTES // 4, dtype=torch.int32, device="cuda"))
        _launch(mq, a, x, qws, cs, mq.MQ_A_FUSED_BF16)
        assert a.s_t() == qa.s_t(), "fused tensor scale differs from the quantizer's"
        if form == "panel":
            assert torch.equal(a.codes, qa.codes), "quantize-once A codes differ from the quantizer's"
            assert torch.equal(a.scales, qa.scales), "quantize-once A scales differ from the quantizer's"
            oa = _check_a_bytes(a, xa, rows, f"cfg{cfg} {projs} panel")
        else:
            oa = _check_a_bytes(qa, xa, rows, f"cfg{cfg} {projs} tile")
        # the whole output against quantize-then-GEMM, bit for bit
        for qw, c in zip(qws, cs):
            c2 = torch.empty_like(c)
            mq.mq_gemm_nvfp4_prefill(qa, None, qw, c2, 0)
            torch.cuda.synchronize()
            assert _same(c, c2), f"{form} fused output differs from quantize-then-GEMM"
            del c2
    for p, c, ow, cols in zip(projs, cs, ows, colss):
        _check_output(c, oa, ow, rows, cols, f"cfg{cfg} {p} ({form})")
    del cs, qws, qa
    _release()


@pytest.mark.parametrize("projs", LAUNCHES, ids=["+".join(g) for g in LAUNCHES])
def test_longctx_quantize_once_launch(projs):
    announce("bench launch cfg3 panel", "+".join(projs))
    _run_launch(3, projs, "panel")


@pytest.mark.parametrize("projs", [("q",), ("gate",)], ids=["q", "gate"])
def test_longctx_per_tile_launch(projs):
    announce("bench launch cfg3 per-tile", "+".join(projs))
    _run_launch(3, projs, "tile")


@pytest.mark.parametrize("projs", LAUNCHES, ids=["+".join(g) for g in LAUNCHES])
def test_70b_slice_launch(projs):
    announce("bench launch cfg5", "+".join(projs))
    _run_launch(5, projs, "separate")


def test_8b_prefill_grouped_kv_launch():
    announce("bench launch cfg2 k+v")
    _run_launch(2, ("k", "v"), "separate")
