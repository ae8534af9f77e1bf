"""GPU parity of lbq_mlp_2bit_i16: bit-exact logits and argmax against the CPU oracle on the
literal workload and on stress sets that exercise wraparound, negative floors, ReLU and the
bit order."""
import numpy as np
import pytest
import torch

import oracle
from packed_weight_gemv_amd import synth
from tests._gpu import to_dev

pytestmark = pytest.mark.gpu


def _run(lbq, codes, dims, x, want_argmax=True):
    lw = [to_dev(lbq.lbq_pack_2bit(c)) for c in codes]
    B = x.shape[0]
    logits = torch.empty((B, dims[-1]), dtype=torch.int16, device="cuda:0")
    am = torch.empty(B, dtype=torch.int32, device="cuda:0") if want_argmax else None
    lbq.lbq_mlp_2bit_i16(lw, dims, to_dev(x), logits, am)
    torch.cuda.synchronize()
    return logits.cpu().numpy(), (am.cpu().numpy() if want_argmax else None)


def _codes_from_values(c):
    c = np.asarray(c, dtype=np.uint8)
    n, k = c.shape
    c4 = c.reshape(n, k // 4, 4)
    return (c4[..., 0] | (c4[..., 1] << 2) | (c4[..., 2] << 4) | (c4[..., 3] << 6)).astype(np.uint8)


def _check(lbq, codes, dims, x):
    lg, am = _run(lbq, codes, dims, x)
    rl, ra = oracle.mlp_2bit(codes, dims, x)
    assert np.array_equal(lg, rl)
    assert np.array_equal(am, ra)
    return lg


def test_literal_workload_bit_exact(lbq):
    dims = list(synth.MLP_DIMS)
    lg = _check(lbq, synth.mlp2bit_layers(), dims, synth.mlp2bit_inputs())
    assert not lg.any()


def test_balanced_codes_bit_exact(lbq):
    dims = list(synth.MLP_DIMS)
    r = np.random.default_rng(41)
    codes = [_codes_from_values(r.integers(1, 4, size=(dims[l + 1], dims[l]))) for l in range(3)]
    lg = _check(lbq, codes, dims, synth.mlp2bit_inputs(batch=1024, extra=41))
    assert lg.any()


def test_wraparound_rows_bit_exact(lbq):
    dims = list(synth.MLP_DIMS)
    codes = [np.zeros((dims[l + 1], dims[l] // 4), dtype=np.uint8) for l in range(3)]
    _check(lbq, codes, dims, synth.mlp2bit_inputs(batch=67, lo=64, hi=128, extra=42))


def test_full_range_inputs_bit_exact(lbq):
    dims = list(synth.MLP_DIMS)
    _check(lbq, synth.mlp2bit_layers(extra=43), dims,
           synth.mlp2bit_inputs(batch=257, lo=-32768, hi=32768, extra=43))


def test_crafted_pre_shift_sums(lbq):
    # one weight +1 on input 0: output = floor(s/4) with s landing on the boundary values
    s = np.array([-32768, 32767, -5, -4, -1, 0, 3, 4, -32767, 32766], dtype=np.int16)
    byte = (2 << 6) | (2 << 4) | (2 << 2) | 3
    codes = [np.full((3, 1), byte, dtype=np.uint8)]
    x = np.zeros((s.size, 4), dtype=np.int16)
    x[:, 0] = s
    lg = _check(lbq, codes, [4, 3], x)
    assert np.array_equal(lg[:, 0].astype(np.int64), s.astype(np.int64) // 4)


def test_one_hot_code_probes(lbq):
    k = 256
    rows = []
    for j in range(k):
        c = np.full(k, 2, dtype=np.uint8)
        c[j] = 3
        rows.append(c)
    codes = [_codes_from_values(np.array(rows))]
    x = synth.mlp2bit_inputs(batch=3, lo=-30000, hi=30000, extra=44)
    lg = _check(lbq, codes, [k, k], x)
    assert np.array_equal(lg.astype(np.int64), x.astype(np.int64) // 4)


@pytest.mark.parametrize("dims,batch", [([260, 100, 12], 7), ([4, 1], 5), ([1024, 1024, 4], 9),
                                        ([64, 64, 64, 64, 64, 64, 64, 64, 3], 33)])
def test_odd_shapes_and_depths(lbq, dims, batch):
    r = np.random.default_rng(46)
    codes = [_codes_from_values(r.integers(1, 4, size=(dims[l + 1], dims[l])))
             for l in range(len(dims) - 1)]
    _check(lbq, codes, dims, synth.mlp2bit_inputs(batch=batch, width=dims[0], lo=-3000, hi=3000,
                                                  extra=47))


@pytest.mark.parametrize("dims", [[1024, 256, 512], [1024, 256, 516]])
def test_codes_at_the_lds_capacity(lbq, dims):
    """Padded codes of exactly 96 KiB (256 x 64 + 512 x 16 dwords: the largest network the
    LDS kernel takes, its codes reaching the top of the workgroup's LDS above the activations)
    and 256 bytes more (the kernel that reads the codes from global memory); 9 vectors, so the
    last workgroup carries one."""
    r = np.random.default_rng(48)
    codes = [_codes_from_values(r.integers(1, 4, size=(dims[l + 1], dims[l])))
             for l in range(len(dims) - 1)]
    _check(lbq, codes, dims, synth.mlp2bit_inputs(batch=9, width=dims[0], lo=-3000, hi=3000,
                                                  extra=49))


def test_argmax_optional(lbq):
    dims = list(synth.MLP_DIMS)
    codes = synth.mlp2bit_layers(extra=48)
    x = synth.mlp2bit_inputs(batch=5, extra=48)
    lg, _ = _run(lbq, codes, dims, x, want_argmax=False)
    rl, _ = oracle.mlp_2bit(codes, dims, x)
    assert np.array_equal(lg, rl)
