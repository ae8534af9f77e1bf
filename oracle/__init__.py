"""Test infrastructure only: the CPU oracle of the packed low-bit GEMV library.

`lbq_oracle.c` is a plain scalar C implementation (exact integers for the 2-bit MLP, IEEE
double precision for the float paths) of what the library computes, written from the pages'
definitions; `exact.py` is an even smaller exact-arithmetic twin (Python integers and
`fractions.Fraction`) for tiny shapes. Both read canonical layouts only and share nothing with
the HIP library. Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of
`bench.py` may import this package.

Parity status of each function is recorded in its docstring.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lbq_oracle.c")
_BUILD = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD, "liblbq_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into oracle/_build/liblbq_oracle.so (plain -O2, no
    fast-math: the IEEE double semantics of the C source are the oracle)."""
    os.makedirs(_BUILD, exist_ok=True)
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
             "-ffp-contract=off", _SRC, "-o", tmp, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32 = ctypes.c_int
    lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f64.restype = ctypes.c_double
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = ctypes.c_double
    lib.oracle_f64_to_bf16_rne.argtypes = [ctypes.c_double]
    lib.oracle_f64_to_bf16_rne.restype = ctypes.c_uint16
    lib.oracle_mlp_2bit.argtypes = [P, P, i32, P, i32, P, P]
    lib.oracle_mlp_2bit.restype = i32
    lib.oracle_gemv_q1g128.argtypes = [P, P, i32, i32, P, i32, P, i32, P, P]
    lib.oracle_gemv_q1g128.restype = None
    lib.oracle_gemv_i4g128.argtypes = [P, P, i32, i32, P, i32, P, i32, P, P]
    lib.oracle_gemv_i4g128.restype = None
    lib.oracle_quant_act_i8g128.argtypes = [P, i32, i32, P, P]
    lib.oracle_quant_act_i8g128.restype = None
    lib.oracle_gemv_i4g128_i8act.argtypes = [P, P, i32, i32, P, P, i32, P, i32, P, P]
    lib.oracle_gemv_i4g128_i8act.restype = None
    lib.oracle_rms_rescale.argtypes = [P, P, i32, i32, ctypes.c_double, P, P]
    lib.oracle_rms_rescale.restype = None
    lib.oracle_round_bf16.argtypes = [P, ctypes.c_size_t, P]
    lib.oracle_round_bf16.restype = None
    lib.oracle_gemv_tern_g160.argtypes = [P, P, i32, i32, P, i32, P, i32, P, P]
    lib.oracle_gemv_tern_g160.restype = None
    lib.oracle_fnv1a32.argtypes = [P, i32]
    lib.oracle_fnv1a32.restype = ctypes.c_uint32
    lib.oracle_z80_normalize.argtypes = [ctypes.c_uint8]
    lib.oracle_z80_normalize.restype = ctypes.c_uint8
    lib.oracle_z80_encode.argtypes = [P, i32, P]
    lib.oracle_z80_encode.restype = None
    lib.oracle_z80_chat.argtypes = [P, P, i32, P, P, i32, i32, i32, P, P]
    lib.oracle_z80_chat.restype = i32
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


# ----------------------------------------------------------------------------------------
# number formats
# ----------------------------------------------------------------------------------------

def f16_to_f64(bits) -> np.ndarray:
    """fp16 bit patterns -> float64 (IEEE binary16 definition, subnormals kept)."""
    lib = _load()
    b = np.asarray(bits, dtype=np.uint16)
    return np.array([lib.oracle_f16_to_f64(int(v)) for v in b.ravel()]).reshape(b.shape)


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 (bfloat16 definition)."""
    lib = _load()
    b = np.asarray(bits, dtype=np.uint16)
    return np.array([lib.oracle_bf16_to_f64(int(v)) for v in b.ravel()]).reshape(b.shape)


def round_bf16(values) -> np.ndarray:
    """float64 -> bf16 bit patterns, round to nearest, ties to even."""
    lib = _load()
    v = _c(values, np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib.oracle_round_bf16(_ptr(v), v.size, _ptr(out))
    return out


# ----------------------------------------------------------------------------------------
# the three formats
# ----------------------------------------------------------------------------------------

def mlp_2bit(layer_codes, dims, x):
    """Z80-uLM-semantics 2-bit MLP, bit-exact (pinned: code map, bit order, wrap, floor
    shift, ReLU placement, argmax ties; see tests/test_oracle_mlp2bit.py).

    layer_codes: list of canonical uint8 [dims[l+1]][dims[l]/4] arrays; x: int16 [B][dims[0]].
    Returns (logits int16 [B][dims[-1]], argmax int32 [B])."""
    lib = _load()
    L = len(layer_codes)
    dims_a = _c(dims, np.int32)
    assert dims_a.size == L + 1
    codes = [_c(c, np.uint8) for c in layer_codes]
    for l, c in enumerate(codes):
        assert c.shape == (dims_a[l + 1], dims_a[l] // 4), (l, c.shape)
    ptrs = (ctypes.c_void_p * L)(*[_ptr(c) for c in codes])
    xa = _c(x, np.int16)
    B = xa.shape[0]
    assert xa.shape == (B, dims_a[0])
    logits = np.zeros((B, int(dims_a[L])), dtype=np.int16)
    am = np.zeros(B, dtype=np.int32)
    rc = lib.oracle_mlp_2bit(ctypes.cast(ptrs, ctypes.c_void_p), _ptr(dims_a), L, _ptr(xa), B,
                             _ptr(logits), _ptr(am))
    if rc != 0:
        raise ValueError("oracle_mlp_2bit: dimension out of range")
    return logits, am


def _gemv(fn, codes, scales, n, k, x, rows):
    lib = _load()
    x2 = _c(x, np.uint16)
    if x2.ndim == 1:
        x2 = x2[None, :]
    B = x2.shape[0]
    assert x2.shape[1] == k
    if rows is None:
        nr = n
        rp = None
    else:
        ra = _c(rows, np.int32)
        nr = ra.size
        rp = _ptr(ra)
    y = np.zeros((B, nr), dtype=np.float64)
    l1 = np.zeros((B, nr), dtype=np.float64)
    getattr(lib, fn)(_ptr(codes), _ptr(scales), n, k, _ptr(x2), B, rp, nr, _ptr(y), _ptr(l1))
    return y, l1


def gemv_q1g128(signs, scales, x, rows=None):
    """Q1_0_g128 GEMV in float64 (pinned: one-hot probes, all-ones/all-zeros sign closed forms,
    dense-dequant library product, exact Fraction brute force; tests/test_oracle_q1.py).

    signs: canonical uint8 [n][k/8]; scales: fp16 bits [n][k/128]; x: bf16 bits [B][k] or [k].
    Returns (y float64 [B][rows], l1 float64 [B][rows])."""
    s = _c(signs, np.uint8)
    n, k8 = s.shape
    k = k8 * 8
    sc = _c(scales, np.uint16)
    assert sc.shape == (n, k // 128)
    return _gemv("oracle_gemv_q1g128", s, sc, n, k, x, rows)


def gemv_i4g128(nib, scales, x, rows=None):
    """INT4 g128 GEMV in float64 (pinned: one-hot probes, all-(-8) closed form, dense-dequant
    library product, exact Fraction brute force; tests/test_oracle_i4.py).

    nib: canonical uint8 [n][k/2]; scales: fp16 bits [n][k/128]; x: bf16 bits [B][k] or [k]."""
    q = _c(nib, np.uint8)
    n, k2 = q.shape
    k = k2 * 2
    sc = _c(scales, np.uint16)
    assert sc.shape == (n, k // 128)
    return _gemv("oracle_gemv_i4g128", q, sc, n, k, x, rows)


def gemv_tern_g160(codes, scales, x, rows=None):
    """Ternary GEMV: codes uint8 [n][k] in {0, 1, 2} (w = t - 1), scales fp16 bits
    [n][ceil(k/160)], x bf16 bits [B][k]. Returns (y [B][rows], l1 [B][rows]) in float64."""
    c = _c(codes, np.uint8)
    n, k = c.shape
    sc = _c(scales, np.uint16)
    assert sc.shape == (n, (k + 159) // 160)
    return _gemv("oracle_gemv_tern_g160", c, sc, n, k, x, rows)


def quant_act_i8g128(x):
    """int8 quantization of bf16 activations per row and per group of 128 (a reading: symmetric
    absmax, d = fp32(max|x|)/127, q = rint(x/d) in fp32, clamped to +-127). Pinned by the
    half-step reconstruction bound, the absmax element mapping to +-127, sign symmetry, exact
    power-of-two scaling and the zero group (tests/test_oracle_i8act.py).

    x: bf16 bits [B][k] or [k]. Returns (q int8 [B][k], d float32 [B][k/128])."""
    lib = _load()
    x2 = _c(x, np.uint16)
    if x2.ndim == 1:
        x2 = x2[None, :]
    B, k = x2.shape
    assert k % 128 == 0
    q = np.zeros((B, k), dtype=np.int8)
    d = np.zeros((B, k // 128), dtype=np.float32)
    lib.oracle_quant_act_i8g128(_ptr(x2), k, B, _ptr(q), _ptr(d))
    return q, d


def gemv_i4g128_i8act(nib, scales, q, d, rows=None):
    """INT4 g128 GEMV on int8-quantized activations: y = sum_g s d sum_j w q with an exact
    integer inner sum (pinned: within the quantization bound of the unquantized product, exact
    equality when every group's activations are integers with absmax 127, exact one-hot;
    tests/test_oracle_i8act.py).

    nib: canonical uint8 [n][k/2]; scales: fp16 bits [n][k/128]; q: int8 [B][k];
    d: float32 [B][k/128]. Returns (y float64 [B][rows], l1 float64 [B][rows])."""
    lib = _load()
    w = _c(nib, np.uint8)
    n, k2 = w.shape
    k = k2 * 2
    sc = _c(scales, np.uint16)
    assert sc.shape == (n, k // 128)
    q2 = _c(q, np.int8)
    d2 = _c(d, np.float32)
    if q2.ndim == 1:
        q2, d2 = q2[None, :], d2[None, :]
    B = q2.shape[0]
    assert q2.shape == (B, k) and d2.shape == (B, k // 128)
    if rows is None:
        nr, rp = n, None
    else:
        ra = _c(rows, np.int32)
        nr, rp = ra.size, _ptr(ra)
    y = np.zeros((B, nr), dtype=np.float64)
    l1 = np.zeros((B, nr), dtype=np.float64)
    lib.oracle_gemv_i4g128_i8act(_ptr(w), _ptr(sc), n, k, _ptr(q2), _ptr(d2), B, rp, nr,
                                 _ptr(y), _ptr(l1))
    return y, l1


def rms_rescale(y, y2=None, eps: float = 1e-6):
    """RMS rescale between GEMVs (a reading; pinned: unit RMS, power-of-two invariance, exact
    Fraction twin; tests/test_oracle_rms.py). y, y2: bf16 bits [B][n].
    Returns (x bf16 bits [B][n], unrounded float64 quotient [B][n])."""
    lib = _load()
    ya = _c(y, np.uint16)
    if ya.ndim == 1:
        ya = ya[None, :]
    B, n = ya.shape
    y2p = None
    if y2 is not None:
        y2a = _c(y2, np.uint16).reshape(B, n)
        y2p = _ptr(y2a)
    out = np.zeros((B, n), dtype=np.uint16)
    ex = np.zeros((B, n), dtype=np.float64)
    lib.oracle_rms_rescale(_ptr(ya), y2p, n, B, float(eps), _ptr(out), _ptr(ex))
    return out, ex


# ----------------------------------------------------------------------------------------
# Z80-uLM character loop (readings of the open points are in oracle/lbq_oracle.c)
# ----------------------------------------------------------------------------------------

Z80_CHARSET = b"\0 ABCDEFGHIJKLMNOPQRSTUVWXYZ0123456789?!"


def fnv1a32(data: bytes) -> int:
    buf = np.frombuffer(bytes(data) or b"\0", dtype=np.uint8).copy()
    return int(_load().oracle_fnv1a32(_ptr(buf), len(data)))


def z80_normalize(c: int) -> int:
    return int(_load().oracle_z80_normalize(c))


def z80_encode(text: bytes) -> np.ndarray:
    """128 trigram buckets (int16) of a text."""
    buf = np.frombuffer(bytes(text) or b"\0", dtype=np.uint8).copy()
    out = np.zeros(128, dtype=np.int16)
    _load().oracle_z80_encode(_ptr(buf), len(text), _ptr(out))
    return out


def z80_chat(layer_codes, dims, prompts, max_reply: int):
    """Generates a reply per prompt (list of bytes). Returns (replies: list of bytes,
    reply bytes uint8 [B][max_reply] zero-padded, lengths int32 [B])."""
    lib = _load()
    L = len(layer_codes)
    dims_a = _c(dims, np.int32)
    codes = [_c(c, np.uint8) for c in layer_codes]
    ptrs = (ctypes.c_void_p * L)(*[_ptr(c) for c in codes])
    B = len(prompts)
    stride = max(1, max((len(p) for p in prompts), default=1))
    pr = np.zeros((B, stride), dtype=np.uint8)
    lens = np.zeros(B, dtype=np.int32)
    for b, p in enumerate(prompts):
        pr[b, :len(p)] = np.frombuffer(bytes(p), dtype=np.uint8)
        lens[b] = len(p)
    rep = np.zeros((B, max(1, max_reply)), dtype=np.uint8)
    rl = np.zeros(B, dtype=np.int32)
    rc = lib.oracle_z80_chat(ctypes.cast(ptrs, ctypes.c_void_p), _ptr(dims_a), L, _ptr(pr),
                             _ptr(lens), stride, B, max_reply, _ptr(rep), _ptr(rl))
    if rc != 0:
        raise ValueError("oracle_z80_chat: bad shape")
    rep = rep[:, :max_reply]
    return [bytes(rep[b, :rl[b]]) for b in range(B)], rep, rl


def argmax_lowest(logits) -> np.ndarray:
    """Index of the maximum of each row, lowest index among ties (plain loop)."""
    a = np.asarray(logits)
    out = np.zeros(a.shape[0], dtype=np.int32)
    for b in range(a.shape[0]):
        best = 0
        for j in range(a.shape[1]):
            if a[b, j] > a[b, best]:
                best = j
        out[b] = best
    return out
