"""GPU parity of lbq_gemv_tern_g160 against the CPU oracle (tolerance: |err| <= 2e-3 * sum|s w x|
per output), on ragged and split-K shapes, batches, the 27B-shaped projections (sampled rows),
exact one-hot probes and exact negation."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from packed_weight_gemv_amd import synth
from tests._gpu import bits, check_within, empty_bf16, to_dev

pytestmark = pytest.mark.gpu


def _run(lbq, m, x, w=None):
    n, k = m.shape
    if w is None:
        w = to_dev(lbq.lbq_pack_tern_g160(m.codes, m.scales))
    y = empty_bf16(x.shape[0], n)
    lbq.lbq_gemv_tern_g160(w, n, k, to_dev(x), y)
    torch.cuda.synchronize()
    return bits(y)


@pytest.mark.parametrize("n,k,batch", [
    (64, 160, 1),        # one group
    (130, 1000, 1),      # ragged rows, ragged last group
    (1, 37, 2),          # one partial group, one row
    (200, 1281, 3),      # a 1-weight last group
    (333, 9000, 5),      # split-K over many super-groups
    (70, 5120, 16),
    (65, 161, 4),
    (257, 2720, 2),      # two full super-groups (17 groups: ragged super-group of one)
])
def test_parity_small_shapes(lbq, n, k, batch):
    m = synth.tern_matrix(n, k, matrix=n + k)
    x = synth.activations(batch, k, workload=synth.W_TERN, matrix=n, extra=batch)
    print(f"tern n={n} k={k} B={batch}", flush=True)
    y = _run(lbq, m, x)
    ref, l1 = oracle.gemv_tern_g160(m.codes, m.scales, x)
    check_within(y, ref, l1, f"tern {n}x{k} B={batch}")


@pytest.mark.parametrize("name", ["q", "k", "gate", "down"])
@pytest.mark.parametrize("batch", [1, 8])
def test_parity_27b_shapes_sampled_rows(lbq, name, batch):
    n, k = synth.stream_shape(name)
    m = synth.tern_matrix(n, k, matrix=synth.STREAM_MATRICES.index(name))
    x = synth.activations(batch, k, workload=synth.W_TERN, extra=100 + batch)
    print(f"tern {name} {n}x{k} B={batch}", flush=True)
    y = _run(lbq, m, x)
    rows = np.unique(np.concatenate([np.arange(0, n, max(1, n // 89)), [n - 1, 63, 64]]))
    rows = rows[rows < n].astype(np.int32)
    ref, l1 = oracle.gemv_tern_g160(m.codes, m.scales, x, rows=rows)
    check_within(y[:, rows], ref, l1, f"tern {name} B={batch}")


def test_one_hot_probes_are_exact(lbq):
    n, k = 96, 330
    m = synth.tern_matrix(n, k, matrix=5)
    w = to_dev(lbq.lbq_pack_tern_g160(m.codes, m.scales))
    one = synth.f32_to_bf16_bits(np.ones(1, dtype=np.float32))[0]
    x = np.zeros((k, k), dtype=np.uint16)
    x[np.arange(k), np.arange(k)] = one
    y = np.concatenate([_run(lbq, m, x[i:i + 16], w) for i in range(0, k, 16)])
    s = oracle.f16_to_f64(m.scales)
    expect = (m.codes.astype(np.float64) - 1) * s[:, np.arange(k) // 160]
    assert np.array_equal(y, oracle.round_bf16(expect.T))


def test_negating_the_activations_negates_exactly(lbq):
    n, k = 256, 3200
    m = synth.tern_matrix(n, k, matrix=6)
    w = to_dev(lbq.lbq_pack_tern_g160(m.codes, m.scales))
    x = synth.activations(3, k, workload=synth.W_TERN, extra=6)
    y1 = _run(lbq, m, x, w)
    y2 = _run(lbq, m, x ^ 0x8000, w)
    nz = (y1 & 0x7FFF) != 0
    assert np.array_equal(y2[nz], y1[nz] ^ 0x8000)


def test_rejects_bad_arguments_and_zero_batch_is_a_no_op(lbq):
    n, k = 64, 320
    m = synth.tern_matrix(n, k, matrix=7)
    w = to_dev(lbq.lbq_pack_tern_g160(m.codes, m.scales))
    x = to_dev(synth.activations(2, k + 2, workload=synth.W_TERN))
    y = torch.full((2, n), 7, dtype=torch.int16, device="cuda:0")
    lib = lbq.load()
    P = ctypes.c_void_p
    assert lib.lbq_gemv_tern_g160(P(w.data_ptr()), n, k, P(x.data_ptr()), P(y.data_ptr()), 0, None) == 0
    assert lib.lbq_gemv_tern_g160(P(w.data_ptr()), n, k, P(x.data_ptr() + 2), P(y.data_ptr()), 2,
                                  None) == -3
    assert lib.lbq_gemv_tern_g160(P(w.data_ptr()), n, 0, P(x.data_ptr()), P(y.data_ptr()), 2, None) == -2
    assert lib.lbq_gemv_tern_g160(P(w.data_ptr()), n, k, P(x.data_ptr()), P(y.data_ptr()), 17,
                                  None) == -2
    torch.cuda.synchronize()
    assert bool((y == 7).all())
