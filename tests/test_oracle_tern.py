"""Pins of the oracle's ternary g160 GEMV: the format size against the page's two model sizes,
an exact Fraction twin on small and ragged shapes, closed forms (all zero, all +1, all -1),
negation, one-hot probes, a dense-dequant library product, and the reduction to the (separately
pinned) Q1 oracle when every weight is +-1 and every scale of a row is equal."""
import os

import numpy as np
import pytest

import oracle
from oracle import exact
from packed_weight_gemv_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _format():
    vals = {}
    with open(os.path.join(GOLD, "tern_format.txt")) as fh:
        for line in fh:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                vals[k] = float(v)
    return vals


def _mat(n, k, seed, probs=(1 / 3, 1 / 3, 1 / 3)):
    r = np.random.default_rng(seed)
    codes = r.choice(3, size=(n, k), p=probs).astype(np.uint8)
    scales = synth.fp16_abs_normal(r, (n, (k + 159) // 160), 0.02)
    return codes, scales


def test_format_size_matches_the_page():
    f = _format()
    g, d, sb = int(f["group"]), int(f["digits_per_byte"]), int(f["scale_bits"])
    assert 3 ** d <= 256 < 3 ** (d + 1)
    bpw = (g // d * 8 + sb) / g
    assert bpw == pytest.approx(1.7)
    assert round(f["one_bit_gb"] * bpw / f["one_bit_bpw"], 1) == f["ternary_gb"]
    # a 128-weight group would need 26 bytes of digits: 6.1 GB, not the page's 5.9
    assert round(f["one_bit_gb"] * ((26 * 8 + sb) / 128) / f["one_bit_bpw"], 1) != f["ternary_gb"]


@pytest.mark.parametrize("n,k", [(3, 160), (2, 200), (2, 37), (1, 480), (2, 321)])
def test_exact_twin(n, k):
    codes, scales = _mat(n, k, 11 + k)
    x = synth.activations(2, k, workload=60, extra=k)
    y, l1 = oracle.gemv_tern_g160(codes, scales, x)
    ex = exact.gemv_tern_g160(codes, scales, x)
    for b in range(2):
        for r in range(n):
            assert y[b, r] == pytest.approx(float(ex[b][r]), rel=1e-12, abs=1e-300)
    assert np.all(l1 >= np.abs(y))


def test_closed_forms():
    n, k = 5, 400
    _, scales = _mat(n, k, 3)
    x = synth.activations(3, k, workload=61)
    xv = oracle.bf16_to_f64(x)
    s = oracle.f16_to_f64(scales)
    gsum = np.stack([xv[:, 160 * g:min(k, 160 * g + 160)].sum(axis=1) for g in range(3)], axis=1)
    plus = gsum @ s.T                                     # [B][n]
    for t, want in ((1, 0 * plus), (2, plus), (0, -plus)):
        y, l1 = oracle.gemv_tern_g160(np.full((n, k), t, np.uint8), scales, x)
        assert np.allclose(y, want, rtol=1e-12, atol=1e-12)
        if t == 1:
            assert not y.any() and not l1.any()


def test_negation_is_exact():
    codes, scales = _mat(7, 1000, 5)
    x = synth.activations(2, 1000, workload=62)
    y1, _ = oracle.gemv_tern_g160(codes, scales, x)
    y2, _ = oracle.gemv_tern_g160(2 - codes, scales, x)
    assert np.array_equal(y2, -y1)


def test_one_hot_probes():
    n, k = 6, 330
    codes, scales = _mat(n, k, 7)
    one = synth.f32_to_bf16_bits(np.ones(1, dtype=np.float32))[0]
    s = oracle.f16_to_f64(scales)
    for j in (0, 159, 160, 329):
        x = np.zeros((1, k), dtype=np.uint16)
        x[0, j] = one
        y, _ = oracle.gemv_tern_g160(codes, scales, x)
        assert np.array_equal(y[0], s[:, j // 160] * (codes[:, j].astype(np.int64) - 1))


def test_dense_dequant_product():
    n, k = 40, 1000
    codes, scales = _mat(n, k, 9, probs=(0.3, 0.4, 0.3))
    x = synth.activations(4, k, workload=63)
    s = oracle.f16_to_f64(scales)
    w = (codes.astype(np.float64) - 1) * s[:, np.arange(k) // 160]
    y, _ = oracle.gemv_tern_g160(codes, scales, x)
    assert np.allclose(y, oracle.bf16_to_f64(x) @ w.T, rtol=1e-12, atol=1e-12)


def test_reduces_to_q1_with_signs_and_equal_scales():
    n, k = 9, 640                                         # a multiple of 128 and of 160
    r = np.random.default_rng(13)
    signs = r.integers(0, 256, size=(n, k // 8), dtype=np.uint8)
    bits = np.unpackbits(signs, axis=1, bitorder="little")
    codes = np.where(bits == 1, 2, 0).astype(np.uint8)
    row_scale = synth.fp16_abs_normal(r, (n, 1), 0.02)
    x = synth.activations(2, k, workload=64)
    yt, _ = oracle.gemv_tern_g160(codes, np.repeat(row_scale, k // 160, axis=1), x)
    yq, _ = oracle.gemv_q1g128(signs, np.repeat(row_scale, k // 128, axis=1), x)
    assert np.allclose(yt, yq, rtol=1e-12, atol=1e-14)
