"""Test infrastructure only: an exact-arithmetic twin of the CPU oracle for tiny shapes.

Python integers (2-bit MLP: accumulate exactly, wrap ONCE modulo 2^16 at the end, which must
equal the C oracle's wrap-per-multiply-accumulate because reduction modulo 2^16 is a ring
homomorphism) and `fractions.Fraction` (float paths: every bf16 / fp16 value is a dyadic
rational, so the GEMV sums are exact). It decodes bit patterns from the formats' definitions
independently of the C oracle, and shares no code with it or with the library.
"""
from __future__ import annotations

from fractions import Fraction


def f16_value(h: int) -> Fraction:
    """IEEE binary16 bit pattern -> exact value (finite patterns only)."""
    sign = -1 if (h >> 15) & 1 else 1
    e = (h >> 10) & 0x1F
    f = h & 0x3FF
    if e == 31:
        raise ValueError("inf/nan")
    if e == 0:
        return sign * Fraction(f, 1 << 24)
    return sign * Fraction(1024 + f) * Fraction(2) ** (e - 25)


def bf16_value(b: int) -> Fraction:
    """bfloat16 bit pattern -> exact value (finite patterns only)."""
    sign = -1 if (b >> 15) & 1 else 1
    e = (b >> 7) & 0xFF
    f = b & 0x7F
    if e == 255:
        raise ValueError("inf/nan")
    if e == 0:
        return sign * Fraction(f) * Fraction(2) ** -133
    return sign * Fraction(128 + f) * Fraction(2) ** (e - 134)


def bf16_rne(v: Fraction) -> int:
    """Exact value -> nearest bf16 bit pattern, ties to even (finite range)."""
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    if a == 0:
        return sign
    # find e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if e >= -126:
        q = a / Fraction(2) ** (e - 7)          # in [128, 256)
        qi = _round_half_even(q)
        if qi == 256:
            qi = 128
            e += 1
        be = e + 127
        if be >= 255:
            return sign | 0x7F80
        return sign | (be << 7) | (qi - 128)
    q = a / Fraction(2) ** -133
    qi = _round_half_even(q)
    return sign | qi


def _round_half_even(q: Fraction) -> int:
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def mlp_2bit(layer_codes, dims, x):
    """Exact integer MLP: exact sums, one wrap modulo 2^16 per neuron, floor(s/4) via Python's
    floor division, ReLU on hidden layers, argmax lowest index. Inputs as nested lists or
    numpy arrays; returns (logits list[list[int]], argmax list[int])."""
    L = len(layer_codes)
    logits, am = [], []
    for xb in x:
        a = [int(v) for v in xb]
        for l in range(L):
            n, k = int(dims[l + 1]), int(dims[l])
            codes = layer_codes[l]
            out = []
            for r in range(n):
                total = 0
                for j in range(k):
                    c = (int(codes[r][j // 4]) >> (2 * (j % 4))) & 3
                    total += (c - 2) * a[j]
                u = total % 65536
                s = u - 65536 if u >= 32768 else u
                h = s // 4
                if l < L - 1:
                    h = max(h, 0)
                out.append(h)
            a = out
        logits.append(a)
        best = 0
        for j, v in enumerate(a):
            if v > a[best]:
                best = j
        am.append(best)
    return logits, am


def gemv_q1g128(signs, scales, x):
    """Exact Q1_0_g128 GEMV: returns y[b][r] as Fractions."""
    n = len(signs)
    k = len(signs[0]) * 8
    out = []
    for xb in x:
        xv = [bf16_value(int(v)) for v in xb]
        row_vals = []
        for r in range(n):
            total = Fraction(0)
            for g in range(k // 128):
                s = f16_value(int(scales[r][g]))
                part = Fraction(0)
                for j in range(128 * g, 128 * g + 128):
                    bit = (int(signs[r][j // 8]) >> (j % 8)) & 1
                    part += xv[j] if bit else -xv[j]
                total += s * part
            row_vals.append(total)
        out.append(row_vals)
    return out


def gemv_i4g128(nib, scales, x):
    """Exact INT4 g128 GEMV: returns y[b][r] as Fractions."""
    n = len(nib)
    k = len(nib[0]) * 2
    out = []
    for xb in x:
        xv = [bf16_value(int(v)) for v in xb]
        row_vals = []
        for r in range(n):
            total = Fraction(0)
            for g in range(k // 128):
                s = f16_value(int(scales[r][g]))
                part = Fraction(0)
                for j in range(128 * g, 128 * g + 128):
                    byte = int(nib[r][j // 2])
                    u = byte & 0xF if j % 2 == 0 else byte >> 4
                    q = u - 16 if u >= 8 else u
                    part += q * xv[j]
                total += s * part
            row_vals.append(total)
        out.append(row_vals)
    return out


def gemv_tern_g160(codes, scales, x):
    """Exact ternary g160 GEMV: codes [n][k] in {0, 1, 2} (w = t - 1), one fp16 scale per 160
    weights along k (the last group may be shorter); returns y[b][r] as Fractions."""
    n = len(codes)
    k = len(codes[0])
    ng = (k + 159) // 160
    out = []
    for xb in x:
        xv = [bf16_value(int(v)) for v in xb]
        row_vals = []
        for r in range(n):
            total = Fraction(0)
            for g in range(ng):
                s = f16_value(int(scales[r][g]))
                part = Fraction(0)
                for j in range(160 * g, min(k, 160 * g + 160)):
                    part += (int(codes[r][j]) - 1) * xv[j]
                total += s * part
            row_vals.append(total)
        out.append(row_vals)
    return out
