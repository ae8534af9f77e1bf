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
