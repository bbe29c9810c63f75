"""GPU parity of mq_quantize_nvfp4 against the oracle: codes, scale bytes and
the tensor scale must be bit-identical."""

import numpy as np
import pytest

import oracle
import workloads
from tests import golden_io
from tests.gpu_util import announce, quantized_host, to_dev_bf16

pytestmark = pytest.mark.gpu


def _mq():
    import fp4_block_scaled_elem_amd as mq
    return mq


def _gpu_quant(bits, given=None):
    import torch
    mq = _mq()
    x = to_dev_bf16(bits)
    q = mq.NVFP4.empty(*bits.shape)
    flags = 0
    if given is not None:
        q.set_s_t(given)
        flags = mq.MQ_SCALE_GIVEN
    mq.mq_quantize_nvfp4(x, q, flags)
    torch.cuda.synchronize()
    return quantized_host(q)


def _check(bits, rows=None, given=None):
    codes, scales, st = _gpu_quant(bits, given)
    ref = oracle.quantize_nvfp4(bits, s_t=given, rows=rows)
    if rows is not None:
        codes, scales = codes[rows], scales[rows]
    assert st == np.float32(ref.s_t).view(np.uint32), (hex(st), float(ref.s_t))
    bad = np.argwhere(codes != ref.codes)
    assert bad.size == 0, f"{len(bad)} code bytes differ, first {bad[:4].tolist()}"
    bad = np.argwhere(scales != ref.scales)
    assert bad.size == 0, f"{len(bad)} scale bytes differ, first {bad[:4].tolist()}"


@pytest.mark.parametrize("name", golden_io.names())
def test_golden(name):
    announce("quantize golden", name)
    g = golden_io.load(name)
    bits = workloads.f32_to_bf16_bits(g["x"])
    codes, scales, st = _gpu_quant(bits)
    assert st == g["s_t_bits"]
    assert np.array_equal(scales, g["scales"])
    assert np.array_equal(codes, g["codes"])


@pytest.mark.parametrize("shape,kind,scale,seed", [
    ((1, 16), "normal", 1.0, 0),
    ((3, 48), "normal", 1.0, 1),
    ((37, 80), "uniform", 7.0, 2),
    ((64, 4096), "lognormal_mixed", 1.0, 3),
    ((129, 272), "normal", 1e-30, 4),
    ((33, 512), "normal", 1e30, 5),
    ((5, 16 * 1021), "lognormal_mixed", 1e-3, 6),
    ((1000, 1008), "normal", 0.02, 7),
])
def test_random_shapes(shape, kind, scale, seed):
    announce("quantize random", shape, kind, scale, seed)
    _check(workloads.random_bf16(shape, seed, scale, kind))


def test_tiny_tensor_scale():
    announce("quantize tiny amax")
    x = np.zeros((2, 32), np.uint16)
    x[0, 0] = 0x0001   # 2^-133
    x[0, 1] = 0x8001
    x[1, 17] = 0x0003
    x[1, 5] = 0x8000   # -0
    _check(x)


def test_zero_tensor_and_zero_groups():
    announce("quantize zeros")
    _check(np.zeros((4, 64), np.uint16))
    b = workloads.random_bf16((8, 64), 8)
    b[2, 16:32] = 0
    b[3, 0:16] = 0x8000
    _check(b)


@pytest.mark.parametrize("given", [1.0, 0.5, 3.0e-5, 7.25])
def test_given_scale(given):
    announce("quantize given", given)
    _check(workloads.random_bf16((17, 96), 9, 2.0), given=np.float32(given))


def test_requantizing_dequantized_values_on_device():
    # DQ(Q(x)) re-quantized by the GPU gives Q(x) back (all group scales
    # normal and s_t a power of two); the expected bytes are the oracle's
    announce("quantize idempotence")
    bits = workloads.random_bf16((64, 256), 10)
    xf = workloads.bf16_bits_to_f32(bits)
    xf[0, 0] = np.float32(2688 * 0.125)
    xf = np.clip(xf, -336, 336).astype(np.float32)
    ref = oracle.quantize_nvfp4(xf)
    assert ref.scales.min() >= 0x08
    xh = oracle.dequantize_nvfp4(ref).astype(np.float32)
    c2, s2, t2 = _gpu_quant(workloads.f32_to_bf16_bits(xh))
    assert np.array_equal(c2, ref.codes) and np.array_equal(s2, ref.scales)
    assert t2 == np.float32(ref.s_t).view(np.uint32)


@pytest.mark.parametrize("cfg,act", [(1, None), (2, "x_qkv"), (2, "x_down")])
def test_config_activations_full(cfg, act):
    announce("quantize config activation", cfg, act)
    bits = workloads.activation(cfg) if act is None else workloads.activation(cfg, act)
    _check(bits)


@pytest.mark.parametrize("cfg,proj", [(1, None), (2, "k"), (2, "gate")])
def test_config_weights_full(cfg, proj):
    announce("quantize config weight", cfg, proj)
    bits = workloads.weight(cfg) if proj is None else workloads.weight(cfg, proj)
    _check(bits)


@pytest.mark.parametrize("cfg,act", [(3, "x_down"), (5, "x_qkv")])
def test_large_activation_sampled_rows(cfg, act):
    announce("quantize large sampled", cfg, act)
    bits = workloads.activation(cfg, act)
    rows = np.random.default_rng(cfg).choice(bits.shape[0], 128, replace=False)
    rows = np.concatenate([rows, [0, bits.shape[0] - 1]])
    _check(bits, rows=rows)


@pytest.mark.parametrize("rows,cols", [(256, 512), (1, 16), (8, 4096), (257, 512), (32, 4112)])
def test_inline_amax_boundary(rows, cols):
    # inputs of at most 2^17 elements are quantized in one launch, every
    # workgroup taking max|x| itself; larger ones run the amax pass first.
    # The largest magnitude sits in the last element; both sides of the
    # limit must equal the oracle byte for byte.
    announce("quantize inline amax", rows, cols)
    import torch
    mq = _mq()
    x = workloads.random_bf16((rows, cols), 81 + rows, 1.0, "normal")
    x[-1, -1] = workloads.f32_to_bf16_bits(np.array([3.0e4], np.float32))[0]
    q = mq.quantize(to_dev_bf16(x))
    torch.cuda.synchronize()
    ref = oracle.quantize_nvfp4(x)
    codes, scales, st = quantized_host(q)
    assert st == int(np.float32(ref.s_t).view(np.uint32))
    assert int(q.rec[1:2].cpu().numpy().view(np.uint32)[0]) == (int(x[-1, -1]) & 0x7FFF) << 16
    assert np.array_equal(scales, ref.scales) and np.array_equal(codes, ref.codes)
