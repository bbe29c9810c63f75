"""The seeded input generators are deterministic and have the stated shapes
and distributions (CPU)."""

import numpy as np

import workloads


def test_cfg1_deterministic_and_shaped():
    x, w = workloads.activation(1), workloads.weight(1)
    assert x.shape == (128, 512) and w.shape == (512, 512)
    assert x.dtype == np.uint16
    workloads._CFG1_CACHE.clear()
    assert workloads.sha256(workloads.activation(1)) == workloads.sha256(x)
    xf = workloads.bf16_bits_to_f32(x)
    col_std = xf.std(axis=0)
    big = np.sort(col_std)[-4:]
    assert np.all(big > 10) and np.sort(col_std)[-5] < 2     # 4 outlier columns x20
    wf = workloads.bf16_bits_to_f32(w)
    assert abs(wf.std() - 0.02) < 0.001


def test_cfg2_outliers_and_weight_sharing_with_decode():
    x = workloads.activation(2, "x_qkv", M=256)
    assert x.shape == (256, 4096)
    xf = workloads.bf16_bits_to_f32(x)
    assert int(np.sum(xf.std(axis=0) > 10)) == 41
    assert workloads.sha256(workloads.weight(4, "k")) == workloads.sha256(workloads.weight(2, "k"))
    assert workloads.weight(2, "down").shape == (4096, 14336)


def test_student_t_unit_variance():
    x = workloads.bf16_bits_to_f32(workloads.activation(3, "x_o", M=512))
    assert abs(x.std() - 1.0) < 0.05
    x5 = workloads.bf16_bits_to_f32(workloads.activation(5, "x_qkv", M=64))
    assert x5.shape == (64, 8192)
    assert int(np.sum(x5.std(axis=0) > 10)) == 41


def test_bf16_rounding_is_nearest_even():
    v = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20], np.float32)
    b = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(v))
    assert list(b) == [1.0, 1.0 + 2 ** -6, -1.0, 1.0 + 2 ** -7]


def test_flops():
    assert workloads.CONFIGS[2].flops() == 2 * 4096 * 4096 * (4096 * 2 + 1024 * 2 + 14336 * 3)
