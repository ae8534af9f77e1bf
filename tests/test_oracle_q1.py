"""Pins of the Q1_0_g128 GEMV oracle: one-hot probes (sign map, bit order, group mapping),
closed forms for all-ones / all-zeros signs, an independent dense-dequant library product, and
exact rational brute force."""
import numpy as np
import pytest
import torch

import oracle
from oracle import exact
from packed_weight_gemv_amd import synth


def _x_f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16) \
        .to(torch.float64).numpy()


def _dense(signs, scales):
    """Dense float64 weights via library routines: unpackbits (LSB first), float16 cast."""
    bits = np.unpackbits(signs, axis=1, bitorder="little").astype(np.float64)
    w = 2.0 * bits - 1.0
    s = scales.view(np.float16).astype(np.float64)
    return w * np.repeat(s, 128, axis=1)


def test_one_hot_probes_pin_sign_map_bit_order_and_groups():
    m = synth.q1_matrix(8, 384, workload=90)
    n, k = m.shape
    one = synth.f32_to_bf16_bits(np.ones(1, dtype=np.float32))[0]
    x = np.zeros((k, k), dtype=np.uint16)
    x[np.arange(k), np.arange(k)] = one
    y, l1 = oracle.gemv_q1g128(m.signs, m.scales, x)
    bits = np.unpackbits(m.signs, axis=1, bitorder="little")            # [n][k]
    s = m.scales.view(np.float16).astype(np.float64)                    # [n][k/128]
    for j in range(k):
        expect = np.where(bits[:, j] == 1, 1.0, -1.0) * s[:, j // 128]
        assert np.array_equal(y[j], expect), j
        assert np.array_equal(l1[j], np.abs(s[:, j // 128]))


def test_all_ones_and_all_zero_signs_give_plus_minus_sum():
    n, k = 3, 512
    x = synth.activations(2, k, workload=91)
    unit = np.full((n, k // 128), 0x3C00, dtype=np.uint16)             # fp16 1.0
    ones = np.full((n, k // 8), 0xFF, dtype=np.uint8)
    zeros = np.zeros((n, k // 8), dtype=np.uint8)
    xs = _x_f64(x).sum(axis=1)
    yp, _ = oracle.gemv_q1g128(ones, unit, x)
    ym, _ = oracle.gemv_q1g128(zeros, unit, x)
    for b in range(2):
        assert np.allclose(yp[b], xs[b], rtol=1e-14, atol=1e-14)
        assert np.allclose(ym[b], -xs[b], rtol=1e-14, atol=1e-14)


def test_matches_dense_dequant_library_product():
    m = synth.q1_matrix(40, 1152, workload=92)
    x = synth.activations(3, 1152, workload=92)
    y, l1 = oracle.gemv_q1g128(m.signs, m.scales, x)
    W = _dense(m.signs, m.scales)
    X = _x_f64(x)
    ref = X @ W.T
    ref_l1 = np.abs(X) @ np.abs(W).T
    assert np.all(np.abs(y - ref) <= 1e-12 * ref_l1)
    assert np.allclose(l1, ref_l1, rtol=1e-13)


def test_row_subset_equals_full_result():
    m = synth.q1_matrix(33, 256, workload=93)
    x = synth.activations(2, 256, workload=93)
    y, l1 = oracle.gemv_q1g128(m.signs, m.scales, x)
    rows = np.array([32, 0, 7, 7, 19], dtype=np.int32)
    ys, l1s = oracle.gemv_q1g128(m.signs, m.scales, x, rows=rows)
    assert np.array_equal(ys, y[:, rows]) and np.array_equal(l1s, l1[:, rows])


def test_exact_rational_brute_force_tiny():
    m = synth.q1_matrix(3, 256, workload=94)
    # include fp16 subnormal scales and a negative scale (the format allows any fp16)
    m.scales[0, 0] = 0x0003
    m.scales[1, 1] = 0x8000 | 0x2E66
    x = synth.activations(2, 256, workload=94)
    y, l1 = oracle.gemv_q1g128(m.signs, m.scales, x)
    ref = exact.gemv_q1g128(m.signs.tolist(), m.scales.tolist(), x.tolist())
    for b in range(2):
        for r in range(3):
            assert abs(y[b, r] - float(ref[b][r])) <= 1e-14 * max(l1[b, r], 1e-300)


def test_planted_transposed_operand_is_caught_by_the_probes():
    """A plausible oracle mistake (reading the sign bits MSB first) fails the one-hot pin."""
    m = synth.q1_matrix(4, 128, workload=95)
    flipped = np.packbits(np.unpackbits(m.signs, axis=1, bitorder="little"), axis=1,
                          bitorder="big")
    one = synth.f32_to_bf16_bits(np.ones(1, dtype=np.float32))[0]
    x = np.zeros((128, 128), dtype=np.uint16)
    x[np.arange(128), np.arange(128)] = one
    y_bad, _ = oracle.gemv_q1g128(flipped, m.scales, x)
    bits = np.unpackbits(m.signs, axis=1, bitorder="little")
    s = m.scales.view(np.float16).astype(np.float64)
    expect = (np.where(bits == 1, 1.0, -1.0) * s[:, :1]).T
    assert not np.array_equal(y_bad, expect)
