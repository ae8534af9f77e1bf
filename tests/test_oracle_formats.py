"""Pins of the oracle's number-format helpers against independent library routines (numpy's
float16, torch's bfloat16) and exact rational arithmetic."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import exact
from tests._golden import read_kv


def test_f16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = oracle.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    finite = np.isfinite(ref)
    assert np.array_equal(mine[finite], ref[finite])
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    assert np.array_equal(np.isinf(mine), np.isinf(ref))


def test_bf16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = oracle.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    finite = np.isfinite(ref)
    assert np.array_equal(mine[finite], ref[finite])
    assert np.array_equal(np.isnan(mine), np.isnan(ref))


def test_bf16_rne_matches_torch_on_float32_values():
    r = np.random.default_rng(7)
    parts = [
        r.standard_normal(20000).astype(np.float32),
        (r.standard_normal(5000) * 1e-39).astype(np.float32),      # bf16 subnormal range
        (r.standard_normal(5000) * 1e37).astype(np.float32),       # near overflow
    ]
    # exact halfway cases: bf16 value + half an ulp, both parities
    base = r.integers(0x0080, 0x7F00, size=4000).astype(np.uint32)
    ties = ((base << 16) | 0x8000).view(np.float32)
    parts.append(ties)
    parts.append(-ties)
    v = np.concatenate(parts)
    mine = oracle.round_bf16(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def test_bf16_rne_matches_exact_rounding_on_doubles():
    r = np.random.default_rng(8)
    v = np.concatenate([r.standard_normal(3000), r.standard_normal(500) * 1e-39,
                        r.standard_normal(500) * 3e38])
    mine = oracle.round_bf16(v)
    for x, m in zip(v, mine):
        assert exact.bf16_rne(Fraction(float(x))) == int(m), x


def test_q1_format_closed_forms():
    g = read_kv("q1_format.txt")
    group = int(g["group"][0])
    bpw = (group * int(g["sign_bits"][0]) + int(g["scale_bits"][0])) / group
    assert bpw == float(g["bits_per_weight"][0])
    # canonical layout sizes: n*k/8 sign bytes + n*k/128 fp16 scales
    n, k = 5120, 5120
    canon_bytes = n * k // 8 + (n * k // group) * 2
    assert canon_bytes * 8 / (n * k) == bpw
    assert round(16 / bpw, 1) == float(g["compression_vs_fp16"][0])


def test_i4_format_closed_forms():
    g = read_kv("i4_format.txt")
    group = int(g["group"][0])
    n, k = 4096, 4096
    canon_bytes = n * k // 2 + (n * k // group) * 2
    assert canon_bytes * 8 / (n * k) == 4 + 16 / group == 4.125
