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


# ------------------------------------------------ single-launch quantizer --
#
# Dynamic-scale inputs of 17 to 64 half-groups (8 elements) per lane of a
# grid of one 512-thread workgroup per CU (on 256 CUs: above 16.8M and up to
# 67.1M elements) are quantized in one launch, each lane keeping up to 32 or
# 48 of its half-groups in registers from the maximum to the encode (up to
# 16 more in LDS), the workgroups meeting at the tensor maximum through
# epoch-tagged slots of the record (rec->flags counts the workgroups'
# starts: it grows by the grid per call).  Other lengths take the amax pass
# and the encode, and leave rec->flags alone.


def _num_cu():
    import torch
    return torch.cuda.get_device_properties(0).multi_processor_count


def _share(rows, cols):
    t = min(_num_cu(), 512) * 512
    return -(-(rows * cols // 8) // t)


def _rec_words(q):
    return q.rec.cpu().numpy().view(np.uint32)


def _sampled_check(q, x, what):
    rows = np.unique(np.concatenate([np.random.default_rng(x.shape[0] + x.shape[1]).choice(x.shape[0], 96),
                                     [0, x.shape[0] - 1]]))
    ref = oracle.quantize_nvfp4(x, rows=rows)
    codes, scales, st = quantized_host(q)
    assert st == int(np.float32(ref.s_t).view(np.uint32)), f"{what}: tensor scale"
    assert np.array_equal(codes[rows], ref.codes), f"{what}: codes"
    assert np.array_equal(scales[rows], ref.scales), f"{what}: scale bytes"
    return ref


@pytest.mark.parametrize("rows,cols", [(4096, 4096), (2999, 7184), (4096, 8192), (4096, 8208), (4096, 11264),
                                       (4096, 12288), (4096, 14336), (4096, 14352), (8192, 8192), (4112, 16384)])
def test_single_launch_lengths(rows, cols):
    # on 256 CUs: 16 (two passes), 21 (ragged), 32, 33 (ragged, 48 kept),
    # 44, 48, 56 (8 held in LDS), 57 (ragged), 64 (16 in LDS) and 65 (two
    # passes) half-groups per lane
    announce("quantize single launch", rows, cols)
    import torch
    mq = _mq()
    x = workloads.random_bf16((rows, cols), 300 + rows + cols, 1.0, "lognormal_mixed")
    q = mq.NVFP4.empty(rows, cols)
    mq.mq_quantize_nvfp4(to_dev_bf16(x), q)
    torch.cuda.synchronize()
    _sampled_check(q, x, f"{rows}x{cols}")
    w = _rec_words(q)
    assert int(w[1]) == int((x & 0x7FFF).max()) << 16, "amax_bits"
    single = 17 <= _share(rows, cols) <= 64
    if single:
        assert int(w[2]) == 0, "no partial maxima are left for a consumer"
        assert int((w[4:4 + _num_cu()] & 0xFFFF0000).max()) == int(w[1]), "the slots reduce to amax"
        assert int(w[3]) == _num_cu(), "every workgroup counts the call once"
    else:
        assert int(w[3]) == 0 and 1 <= int(w[2]) <= mq.MQ_AMAX_PARTS, "the amax pass's partial maxima"
    assert mq.mq_check_quant_gave_up() == 0


def test_single_launch_forced_give_up():
    # With no polls allowed every workgroup stops waiting at once and reads
    # the whole input for its maximum: the same bytes, only slower.
    announce("quantize single launch, forced give-up")
    import torch
    mq = _mq()
    mq.mq_check_quant_gave_up()
    x = workloads.random_bf16((4096, 6144), 71, 3.0, "normal")
    assert 17 <= _share(*x.shape) <= 64
    q = mq.NVFP4.empty(*x.shape)
    old = mq.mq_check_set_quant_spin_limit(0)
    try:
        mq.mq_quantize_nvfp4(to_dev_bf16(x), q)
        torch.cuda.synchronize()
    finally:
        mq.mq_check_set_quant_spin_limit(old)
    assert mq.mq_check_quant_gave_up() == _num_cu()
    _sampled_check(q, x, "forced give-up")
    # and the next call on the same record waits normally again
    y = workloads.random_bf16((4096, 6144), 72, 0.5, "normal")
    mq.mq_quantize_nvfp4(to_dev_bf16(y), q)
    torch.cuda.synchronize()
    assert mq.mq_check_quant_gave_up() == 0
    _sampled_check(q, y, "after forced give-up")


def test_single_launch_epochs_on_one_record():
    # Successive calls on one record, each with a smaller maximum than the
    # last (a slot read from an earlier call would raise the scale), with a
    # producer's partial maxima written into the same record in between.
    announce("quantize single launch, repeated calls on one record")
    import torch
    mq = _mq()
    rows, cols = 4096, 5120
    assert 17 <= _share(rows, cols) <= 64
    q = mq.NVFP4.empty(rows, cols)
    g = to_dev_bf16(workloads.random_bf16((cols,), 9, 1.0, "normal"))
    y = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    calls = 0
    for i in range(5):
        x = workloads.random_bf16((rows, cols), 400 + i, 64.0 / 2 ** i, "normal")
        mq.mq_quantize_nvfp4(to_dev_bf16(x), q)
        calls += 1
        torch.cuda.synchronize()
        _sampled_check(q, x, f"call {i}")
        if i % 2 == 0:
            # partial maxima (untagged) over the slots, then their consumer
            mq.mq_rmsnorm_amax(to_dev_bf16(x), g, y, q)
            mq.mq_quantize_nvfp4(y, q, mq.MQ_SCALE_PARTIALS)
            torch.cuda.synchronize()
    assert int(_rec_words(q)[3]) == calls * _num_cu()
    assert mq.mq_check_quant_gave_up() == 0
