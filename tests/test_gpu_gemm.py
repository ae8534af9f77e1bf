"""GPU parity of the many-row products lbq_gemm_q1g128 / lbq_gemm_i4g128 (matrix cores) against
the CPU oracle (tolerance: |err| <= 2e-3 * sum|s w x| per output), exact one-hot probes and
negation, and the split-K and ragged-edge paths."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from packed_weight_gemv_amd import synth
from tests._gpu import bits, check_within, empty_bf16, to_dev

pytestmark = pytest.mark.gpu


def _pack(lbq, fmt, m):
    return to_dev(lbq.lbq_pack_q1g128(m.signs, m.scales) if fmt == "q1"
                  else lbq.lbq_pack_i4g128(m.nib, m.scales))


def _matrix(fmt, n, k, **kw):
    return synth.q1_matrix(n, k, **kw) if fmt == "q1" else synth.i4_matrix(n, k, **kw)


def _oracle(fmt, m, x, rows=None):
    if fmt == "q1":
        return oracle.gemv_q1g128(m.signs, m.scales, x, rows=rows)
    return oracle.gemv_i4g128(m.nib, m.scales, x, rows=rows)


def _gemm(lbq, fmt, w, n, k, x):
    y = empty_bf16(x.shape[0], n)
    (lbq.lbq_gemm_q1g128 if fmt == "q1" else lbq.lbq_gemm_i4g128)(w, n, k, to_dev(x), y)
    torch.cuda.synchronize()
    return bits(y)


@pytest.mark.parametrize("fmt", ["q1", "i4"])
@pytest.mark.parametrize("n,k,m", [
    (130, 1152, 33),     # ragged rows (not a multiple of 64 or 256), ragged super-group, 2 row blocks
    (64, 128, 1),        # one group, one row
    (1, 256, 100),       # a single output row, four activation blocks with a ragged one
    (200, 2176, 70),
    (333, 9216, 5),      # split-K over many groups
    (1000, 1024, 64),
    (512, 4096, 97),
    (300, 2176, 150),    # 128-row activation tiles with a ragged last tile
])
def test_parity_small_shapes(lbq, fmt, n, k, m):
    mat = _matrix(fmt, n, k, workload=40, matrix=n + m)
    x = synth.activations(m, k, workload=40, matrix=n, extra=m)
    print(f"gemm {fmt} n={n} k={k} m={m}", flush=True)
    y = _gemm(lbq, fmt, _pack(lbq, fmt, mat), n, k, x)
    ref, l1 = _oracle(fmt, mat, x)
    check_within(y, ref, l1, f"gemm {fmt} {n}x{k} m={m}")


@pytest.mark.parametrize("fmt,n,k,m", [
    ("q1", 17408, 5120, 32), ("q1", 17408, 5120, 512), ("q1", 5120, 17408, 128),
    ("q1", 5120, 5120, 256),
    ("i4", 4096, 4096, 64), ("i4", 12288, 4096, 512), ("i4", 4096, 12288, 32),
])
def test_parity_full_size_sampled_rows(lbq, fmt, n, k, m):
    wl = synth.W_Q1_MLP if fmt == "q1" else synth.W_I4_LAYER
    mat = _matrix(fmt, n, k, workload=wl, matrix=n + k)
    x = synth.activations(m, k, workload=wl, matrix=n + k, extra=1000 + m)
    print(f"gemm {fmt} full n={n} k={k} m={m}", flush=True)
    y = _gemm(lbq, fmt, _pack(lbq, fmt, mat), n, k, x)
    rows = np.unique(np.concatenate([np.arange(0, n, max(1, n // 61)), [n - 1, 63, 64, 255, 256]]))
    rows = rows[rows < n].astype(np.int32)
    sel = np.unique(np.concatenate([np.arange(0, m, max(1, m // 24)), [m - 1]]))
    ref, l1 = _oracle(fmt, mat, x[sel], rows=rows)
    check_within(y[sel][:, rows], ref, l1, f"gemm {fmt} {n}x{k} m={m}")


@pytest.mark.parametrize("fmt", ["q1", "i4"])
def test_one_hot_probes_are_exact(lbq, fmt):
    n, k = 96, 384
    mat = _matrix(fmt, n, k, workload=41)
    w = _pack(lbq, fmt, mat)
    one = synth.f32_to_bf16_bits(np.ones(1, dtype=np.float32))[0]
    x = np.zeros((k, k), dtype=np.uint16)
    x[np.arange(k), np.arange(k)] = one
    y = _gemm(lbq, fmt, w, n, k, x)
    scales = oracle.f16_to_f64(mat.scales)
    if fmt == "q1":
        wv = np.where(np.unpackbits(mat.signs, axis=1, bitorder="little") == 1, 1.0, -1.0)
    else:
        lo = (mat.nib & 0xF).astype(np.int64)
        hi = (mat.nib >> 4).astype(np.int64)
        q = np.empty((n, k), dtype=np.int64)
        q[:, 0::2], q[:, 1::2] = lo, hi
        wv = np.where(q >= 8, q - 16, q).astype(np.float64)
    expect = wv * scales[:, np.arange(k) // 128]
    assert np.array_equal(y, oracle.round_bf16(expect.T))


@pytest.mark.parametrize("fmt", ["q1", "i4"])
def test_negating_the_activations_negates_exactly(lbq, fmt):
    n, k, m = 256, 3072, 40
    mat = _matrix(fmt, n, k, workload=42)
    w = _pack(lbq, fmt, mat)
    x = synth.activations(m, k, workload=42)
    y1 = _gemm(lbq, fmt, w, n, k, x)
    y2 = _gemm(lbq, fmt, w, n, k, x ^ 0x8000)
    nz = (y1 & 0x7FFF) != 0
    assert np.array_equal(y2[nz], y1[nz] ^ 0x8000)


@pytest.mark.parametrize("fmt", ["q1", "i4"])
def test_agrees_with_the_gemv_path(lbq, fmt):
    n, k, m = 320, 5120, 16
    mat = _matrix(fmt, n, k, workload=43)
    w = _pack(lbq, fmt, mat)
    x = synth.activations(m, k, workload=43)
    y = _gemm(lbq, fmt, w, n, k, x)
    yv = empty_bf16(m, n)
    (lbq.lbq_gemv_q1g128 if fmt == "q1" else lbq.lbq_gemv_i4g128)(w, n, k, to_dev(x), yv)
    torch.cuda.synchronize()
    ref, l1 = _oracle(fmt, mat, x)
    check_within(y, ref, l1, "gemm")
    check_within(bits(yv), ref, l1, "gemv")


def test_zero_rows_is_a_no_op_and_misaligned_x_is_rejected(lbq):
    n, k = 64, 256
    mat = _matrix("q1", n, k, workload=44)
    w = _pack(lbq, "q1", mat)
    y = torch.full((4, n), 7, dtype=torch.int16, device="cuda:0")
    x = to_dev(synth.activations(4, k + 8, workload=44))
    lib = lbq.load()
    st = lib.lbq_gemm_q1g128(ctypes.c_void_p(w.data_ptr()), n, k, ctypes.c_void_p(x.data_ptr()),
                             ctypes.c_void_p(y.data_ptr()), 0, None)
    assert st == 0
    st = lib.lbq_gemm_q1g128(ctypes.c_void_p(w.data_ptr()), n, k, ctypes.c_void_p(x.data_ptr() + 8),
                             ctypes.c_void_p(y.data_ptr()), 4, None)
    assert st == -3   # LBQ_E_ALIGN: x must be 16-byte aligned
    torch.cuda.synchronize()
    assert bool((y == 7).all())
