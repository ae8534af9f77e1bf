"""GPU parity of lbq_gemv_i4g128 against the CPU oracle (tolerance: |err| <= 2e-3 * sum|s q x|),
plus exact one-hot probes and bitwise metamorphic properties."""
import numpy as np
import pytest
import torch

import oracle
from packed_weight_gemv_amd import synth
from tests._gpu import bits, check_within, empty_bf16, to_dev

pytestmark = pytest.mark.gpu


def _run(lbq, m, x):
    n, k = m.shape
    w = to_dev(lbq.lbq_pack_i4g128(m.nib, m.scales))
    y = empty_bf16(x.shape[0], n)
    lbq.lbq_gemv_i4g128(w, n, k, to_dev(x), y)
    torch.cuda.synchronize()
    return bits(y)


@pytest.mark.parametrize("n,k", [(130, 1152), (64, 128), (1, 256), (200, 2176)])
def test_parity_small_shapes_with_ragged_tails(lbq, n, k):
    m = synth.i4_matrix(n, k, workload=30, matrix=n)
    x = synth.activations(1, k, workload=30, matrix=n)
    y = _run(lbq, m, x)
    ref, l1 = oracle.gemv_i4g128(m.nib, m.scales, x)
    check_within(y, ref, l1, f"i4 {n}x{k}")


@pytest.mark.parametrize("batch", [1, 2, 3, 8, 16])
def test_parity_batches(lbq, batch):
    n, k = 192, 2048
    m = synth.i4_matrix(n, k, workload=31)
    x = synth.activations(batch, k, workload=31, extra=batch)
    y = _run(lbq, m, x)
    ref, l1 = oracle.gemv_i4g128(m.nib, m.scales, x)
    check_within(y, ref, l1, f"i4 batch {batch}")


@pytest.mark.parametrize("n,k,batch", [(130, 1024, 5), (64, 128, 3), (333, 9216, 16),
                                         (65, 3200, 7), (1, 384, 2)])
def test_parity_matrix_core_batches_ragged(lbq, n, k, batch):
    """2-16 vectors run on the matrix cores: one k slice (k <= 1024), many slices, a last
    super-group with one group, rows past a tile boundary, a single row."""
    m = synth.i4_matrix(n, k, workload=33, matrix=n + k)
    x = synth.activations(batch, k, workload=33, matrix=n + k, extra=batch)
    y = _run(lbq, m, x)
    ref, l1 = oracle.gemv_i4g128(m.nib, m.scales, x)
    check_within(y, ref, l1, f"i4 {n}x{k} B={batch}")


@pytest.mark.parametrize("name,n,k", [(nm, n, k) for nm, n, k in synth.I4_SHAPES
                                      if nm in ("q", "k", "gate", "down")])
@pytest.mark.parametrize("batch", [1, 8])
def test_parity_qwen3_8b_shapes_sampled_rows(lbq, name, n, k, batch):
    m = synth.i4_matrix(n, k, workload=synth.W_I4_LAYER, matrix=synth.STREAM_MATRICES.index(name))
    x = synth.activations(batch, k, workload=synth.W_I4_LAYER, extra=batch)
    y = _run(lbq, m, x)
    rows = np.unique(np.concatenate([np.arange(0, n, max(1, n // 89)), [n - 1]])).astype(np.int32)
    ref, l1 = oracle.gemv_i4g128(m.nib, m.scales, x, rows=rows)
    check_within(y[:, rows], ref, l1, f"i4 {name} B={batch}")


def test_one_hot_probes_are_exact(lbq):
    n, k = 64, 256
    m = synth.i4_matrix(n, k, workload=32)
    one = synth.f32_to_bf16_bits(np.ones(1, dtype=np.float32))[0]
    lo = (m.nib & 0xF).astype(np.int64)
    hi = (m.nib >> 4).astype(np.int64)
    q = np.stack([lo, hi], axis=-1).reshape(n, k)
    q = np.where(q >= 8, q - 16, q)
    for j in range(0, k, 5):
        x = np.zeros((1, k), dtype=np.uint16)
        x[0, j] = one
        y = _run(lbq, m, x)
        expect = q[:, j] * oracle.f16_to_f64(m.scales[:, j // 128])
        assert np.array_equal(y[0], oracle.round_bf16(expect)), j


def test_all_codes_minus_eight(lbq):
    n, k = 64, 1024
    m = synth.i4_matrix(n, k, workload=33)
    m.nib[:] = 0x88
    x = synth.activations(2, k, workload=33)
    y = _run(lbq, m, x)
    ref, l1 = oracle.gemv_i4g128(m.nib, m.scales, x)
    check_within(y, ref, l1, "i4 all -8")


def test_power_of_two_input_scaling_is_exact_and_deterministic(lbq):
    n, k = 128, 4096
    m = synth.i4_matrix(n, k, workload=34)
    x = synth.activations(1, k, workload=34)
    x2 = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(x) * np.float32(0.5))
    y1 = _run(lbq, m, x)
    y2 = _run(lbq, m, x2)
    assert np.array_equal(oracle.bf16_to_f64(y2), 0.5 * oracle.bf16_to_f64(y1))
    assert np.array_equal(_run(lbq, m, x), y1)


@pytest.mark.parametrize("batch", [2, 4, 16])
def test_parity_batches_with_rows_not_16_byte_aligned(lbq, batch):
    # x at a 4-byte but not 16-byte aligned address: the per-row lookup kernels (aligned
    # batches take the matrix-core product)
    n, k = 192, 2176
    m = synth.i4_matrix(n, k, workload=24)
    x = synth.activations(batch, k, workload=24, extra=batch)
    buf = torch.zeros(batch * k + 8, dtype=torch.int16, device="cuda:0")
    xv = buf[2:2 + batch * k].view(batch, k)
    assert xv.data_ptr() % 16 == 4
    xv.copy_(to_dev(x))
    w = to_dev(lbq.lbq_pack_i4g128(m.nib, m.scales))
    y = empty_bf16(batch, n)
    lbq.lbq_gemv_i4g128(w, n, k, xv, y)
    torch.cuda.synchronize()
    ref, l1 = oracle.gemv_i4g128(m.nib, m.scales, x)
    check_within(bits(y), ref, l1, f"i4 unaligned batch {batch}")
