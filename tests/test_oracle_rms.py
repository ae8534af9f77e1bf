"""Pins of the RMS-rescale oracle (a reading: the pages name no formula): unit RMS of the
output, invariance under power-of-two scaling, an independent float64 library computation, and
exact rounding of the quotient."""
from fractions import Fraction

import numpy as np
import torch

import oracle
from oracle import exact
from packed_weight_gemv_amd import synth


def _f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16) \
        .to(torch.float64).numpy()


def test_output_has_unit_rms():
    y = synth.activations(3, 5120, workload=80)
    x, q = oracle.rms_rescale(y, eps=1e-6)
    rms = np.sqrt((_f64(x) ** 2).mean(axis=1))
    assert np.all(np.abs(rms - 1.0) < 2 ** -8)
    assert np.allclose(np.sqrt((q ** 2).mean(axis=1)), 1.0, rtol=1e-6)


def test_power_of_two_scaling_invariance():
    y = synth.activations(2, 1024, workload=81)
    y4 = synth.f32_to_bf16_bits((_f64(y) * 4.0).astype(np.float32))
    a, _ = oracle.rms_rescale(y, eps=0.0)
    b, _ = oracle.rms_rescale(y4, eps=0.0)
    assert np.array_equal(a, b)


def test_matches_library_float64_and_exact_rounding():
    g = synth.activations(2, 768, workload=82)
    u = synth.activations(2, 768, workload=83)
    x, q = oracle.rms_rescale(g, u, eps=1e-6)
    h = _f64(g) * _f64(u)
    ref = h / np.sqrt((h ** 2).mean(axis=1, keepdims=True) + 1e-6)
    assert np.allclose(q, ref, rtol=1e-14, atol=0)
    for b in range(2):
        for j in range(0, 768, 7):
            assert exact.bf16_rne(Fraction(float(q[b, j]))) == int(x[b, j])


def test_zero_vector_stays_zero():
    y = np.zeros((1, 256), dtype=np.uint16)
    x, q = oracle.rms_rescale(y, eps=1e-6)
    assert not x.any() and not q.any()


# ---- the product branch h = y * y2 (feeds every down GEMV of the decode step) --------------
# These fix h by mathematics rather than by restating the formula: a unit second factor, the
# symmetry of the product, power-of-two factors, and a closed form whose output is known exactly.

BF16_ONE, BF16_FOUR, BF16_QUARTER = 0x3F80, 0x4080, 0x3E80


def test_product_with_unit_factor_is_the_single_input_rescale():
    y = synth.activations(2, 1536, workload=84)
    ones = np.full_like(y, BF16_ONE)
    a, qa = oracle.rms_rescale(y, eps=1e-6)
    b, qb = oracle.rms_rescale(y, ones, eps=1e-6)
    assert np.array_equal(a, b) and np.array_equal(qa, qb)


def test_product_is_symmetric_in_its_factors():
    g = synth.activations(2, 1024, workload=85)
    u = synth.activations(2, 1024, workload=86)
    a, qa = oracle.rms_rescale(g, u, eps=1e-6)
    b, qb = oracle.rms_rescale(u, g, eps=1e-6)
    assert np.array_equal(a, b) and np.array_equal(qa, qb)


def test_power_of_two_second_factor_leaves_output_unchanged():
    y = synth.activations(2, 640, workload=87)
    a, _ = oracle.rms_rescale(y, eps=0.0)
    for c in (BF16_FOUR, BF16_QUARTER):
        b, _ = oracle.rms_rescale(y, np.full_like(y, c), eps=0.0)
        assert np.array_equal(a, b)


def test_product_closed_form_signs():
    # |y| = 3 and |y2| = 2 everywhere with independent signs: h = +-6, mean(h^2) = 36, so with
    # eps = 0 every output is exactly sign(y) * sign(y2). Dropping either factor, or using one in
    # place of the other, flips the outputs where that factor is negative.
    r = np.random.default_rng([0x1B0, 88])
    sy = r.integers(0, 2, size=(2, 512)).astype(np.uint16)
    s2 = r.integers(0, 2, size=(2, 512)).astype(np.uint16)
    y = (0x4040 | (sy << 15)).astype(np.uint16)        # +-3.0
    y2 = (0x4000 | (s2 << 15)).astype(np.uint16)       # +-2.0
    x, q = oracle.rms_rescale(y, y2, eps=0.0)
    want = np.where(sy ^ s2, -1.0, 1.0)
    assert np.array_equal(q, want)
    assert np.array_equal(x, np.where(sy ^ s2, 0xBF80, 0x3F80).astype(np.uint16))
    # with eps > 0 the closed form is h / sqrt(36 + eps)
    x, q = oracle.rms_rescale(y, y2, eps=0.25)
    assert np.allclose(q, want * 6.0 / np.sqrt(36.25), rtol=1e-15, atol=0)
