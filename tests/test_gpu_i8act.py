"""GPU parity of the int8-activation path: lbq_quant_act_i8g128 bit-exact to the oracle's codes and
scales, and lbq_gemv_i4g128_act_i8 within 2e-3 * sum|s d w q| of the oracle's integer-dot product
(the integer group sums are exact on both sides; only the fp32 accumulation over groups differs)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from packed_weight_gemv_amd import synth
from tests._gpu import bits, check_within, empty_bf16, to_dev

pytestmark = pytest.mark.gpu


def _quant(lbq, x):
    B, k = x.shape
    q = torch.empty((B, k), dtype=torch.int8, device="cuda:0")
    d = torch.empty((B, k // 128), dtype=torch.float32, device="cuda:0")
    lbq.lbq_quant_act_i8g128(to_dev(x), q, d)
    torch.cuda.synchronize()
    return q.cpu().numpy(), d.cpu().numpy()


def _gemv(lbq, m, x, w=None):
    n, k = m.shape
    if w is None:
        w = to_dev(lbq.lbq_pack_i4g128(m.nib, m.scales))
    y = empty_bf16(x.shape[0], n)
    lbq.lbq_gemv_i4g128_act_i8(w, n, k, to_dev(x), y)
    torch.cuda.synchronize()
    return bits(y)


def _ref(m, x, rows=None):
    q, d = oracle.quant_act_i8g128(x)
    return oracle.gemv_i4g128_i8act(m.nib, m.scales, q, d, rows=rows)


@pytest.mark.parametrize("batch,k", [(1, 128), (3, 1152), (16, 4096), (2, 12288), (5, 640)])
def test_quantization_is_bit_exact(lbq, batch, k):
    x = synth.activations(batch, k, workload=90, extra=batch * k)
    print(f"quant B={batch} k={k}", flush=True)
    q, d = _quant(lbq, x)
    qr, dr = oracle.quant_act_i8g128(x)
    assert np.array_equal(q, qr)
    assert np.array_equal(d.view(np.uint32), dr.view(np.uint32))


def test_quantization_special_groups(lbq):
    k = 128 * 5
    x = synth.activations(2, k, workload=91)
    x[0, 0:128] = 0                                          # zero group: d = 0, q = 0
    x[0, 128:256] = 0x8000                                   # negative zeros
    r = np.random.default_rng(91)
    ties = (r.integers(-120, 120, size=128) + 0.5).astype(np.float32)
    ties[5] = 127.0                                          # d = 1: every other value a tie
    x[1, 0:128] = synth.f32_to_bf16_bits(ties)
    x[1, 128:256] = synth.f32_to_bf16_bits(np.full(128, -3.0, np.float32))   # all at -absmax
    tiny = synth.bf16_bits_to_f32(x[1, 256:384]) * np.float32(1e-30)
    x[1, 256:384] = synth.f32_to_bf16_bits(tiny.astype(np.float32))
    q, d = _quant(lbq, x)
    qr, dr = oracle.quant_act_i8g128(x)
    assert np.array_equal(q, qr) and np.array_equal(d.view(np.uint32), dr.view(np.uint32))
    assert d[0, 0] == 0 and d[0, 1] == 0 and not q[0, :256].any()
    # ties round to even
    assert np.array_equal(q[1, :128].astype(np.float64), np.where(np.arange(128) == 5, 127.0,
                                                                  np.rint(ties)))
    assert np.all(q[1, 128:256] == -127)


@pytest.mark.parametrize("n,k,batch", [
    (64, 128, 1),        # one group
    (130, 1152, 3),      # ragged rows, ragged super-group
    (1, 256, 2),         # one output row
    (200, 2176, 7),
    (333, 9216, 5),      # split-K over many super-groups
    (1000, 1024, 16),
    (70, 4096, 9),
])
def test_parity_small_shapes(lbq, n, k, batch):
    m = synth.i4_matrix(n, k, workload=92, matrix=n + batch)
    x = synth.activations(batch, k, workload=92, matrix=n, extra=batch)
    print(f"i8act gemv n={n} k={k} B={batch}", flush=True)
    y = _gemv(lbq, m, x)
    ref, l1 = _ref(m, x)
    check_within(y, ref, l1, f"i8act {n}x{k} B={batch}")


@pytest.mark.parametrize("name,n,k", [(nm, n, k) for nm, n, k in synth.I4_SHAPES
                                      if nm in ("q", "gate", "down")])
@pytest.mark.parametrize("batch", [1, 16])
def test_parity_qwen3_8b_shapes_sampled_rows(lbq, name, n, k, batch):
    m = synth.i4_matrix(n, k, workload=synth.W_I4_LAYER, matrix=synth.STREAM_MATRICES.index(name))
    x = synth.activations(batch, k, workload=synth.W_I4_LAYER, extra=100 + batch)
    print(f"i8act gemv {name} {n}x{k} B={batch}", flush=True)
    y = _gemv(lbq, m, x)
    rows = np.unique(np.concatenate([np.arange(0, n, max(1, n // 89)), [n - 1]])).astype(np.int32)
    ref, l1 = _ref(m, x, rows=rows)
    check_within(y[:, rows], ref, l1, f"i8act {name} B={batch}")


def test_one_hot_127_is_exact(lbq):
    n, k = 64, 384
    m = synth.i4_matrix(n, k, workload=93)
    w = to_dev(lbq.lbq_pack_i4g128(m.nib, m.scales))
    v = synth.f32_to_bf16_bits(np.array([127.0], dtype=np.float32))[0]
    x = np.zeros((k, k), dtype=np.uint16)
    x[np.arange(k), np.arange(k)] = v
    y = np.concatenate([_gemv(lbq, m, x[i:i + 16], w) for i in range(0, k, 16)])
    lo = (m.nib & 0xF).astype(np.int64)
    hi = (m.nib >> 4).astype(np.int64)
    q = np.empty((n, k), dtype=np.int64)
    q[:, 0::2], q[:, 1::2] = lo, hi
    wv = np.where(q >= 8, q - 16, q).astype(np.float64)
    expect = wv * oracle.f16_to_f64(m.scales)[:, np.arange(k) // 128] * 127.0
    assert np.array_equal(y, oracle.round_bf16(expect.T))


def test_agrees_with_the_float_path_on_exactly_quantized_activations(lbq):
    # integers in [-127, 127] with 127 in every group quantize exactly (d = 1, q = x)
    n, k, B = 256, 3072, 4
    m = synth.i4_matrix(n, k, workload=94)
    r = np.random.default_rng(94)
    xi = r.integers(-127, 128, size=(B, k))
    xi[:, ::128] = 127
    x = synth.f32_to_bf16_bits(xi.astype(np.float32))
    y8 = _gemv(lbq, m, x)
    ref, l1 = oracle.gemv_i4g128(m.nib, m.scales, x)
    check_within(y8, ref, l1, "i8act vs float oracle")


def test_rejects_bad_arguments_and_zero_batch_is_a_no_op(lbq):
    n, k = 64, 256
    m = synth.i4_matrix(n, k, workload=95)
    w = to_dev(lbq.lbq_pack_i4g128(m.nib, m.scales))
    x = to_dev(synth.activations(2, k + 2, workload=95))
    y = torch.full((2, n), 7, dtype=torch.int16, device="cuda:0")
    lib = lbq.load()
    P = ctypes.c_void_p
    assert lib.lbq_gemv_i4g128_act_i8(P(w.data_ptr()), n, k, P(x.data_ptr()), P(y.data_ptr()),
                                      0, None) == 0
    assert lib.lbq_gemv_i4g128_act_i8(P(w.data_ptr()), n, k, P(x.data_ptr() + 2),
                                      P(y.data_ptr()), 2, None) == -3
    assert lib.lbq_gemv_i4g128_act_i8(P(w.data_ptr()), n, k + 64, P(x.data_ptr()),
                                      P(y.data_ptr()), 2, None) == -2
    q = torch.empty((2, k), dtype=torch.int8, device="cuda:0")
    d = torch.empty((2, 2), dtype=torch.float32, device="cuda:0")
    assert lib.lbq_quant_act_i8g128(P(x.data_ptr()), 200, 2, P(q.data_ptr()), P(d.data_ptr()),
                                    None) == -2
    assert lib.lbq_quant_act_i8g128(P(x.data_ptr()), k, 2, P(q.data_ptr()), P(x.data_ptr()),
                                    None) == -5
    torch.cuda.synchronize()
    assert bool((y == 7).all())
