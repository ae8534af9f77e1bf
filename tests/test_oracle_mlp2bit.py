"""Pins of the 2-bit integer MLP oracle (Z80-uLM semantics) to what the page and arithmetic fix:
the code map, the bit order of the unpack listing, floor shifting, ReLU placement, 16-bit
wraparound and the degenerate literal workload."""
import numpy as np
import pytest

import oracle
from oracle import exact
from packed_weight_gemv_amd import synth
from tests._golden import read_kv, read_pairs


def _one_layer(codes_byte_rows, x):
    """1-layer MLP (no ReLU: it is the output layer) with k = 4 * len(row)."""
    codes = np.array(codes_byte_rows, dtype=np.uint8)
    n, kb = codes.shape
    return oracle.mlp_2bit([codes], [4 * kb, n], np.array(x, dtype=np.int16))


def test_code_map_matches_the_page():
    # weight of code c is probed with input 400 on slot 0, every other slot code 2 (weight 0)
    for code, weight in ((int(a), int(b)) for a, b in read_pairs("z80_code_map.txt")):
        byte = (2 << 6) | (2 << 4) | (2 << 2) | code
        logits, _ = _one_layer([[byte]], [[400, 0, 0, 0]])
        assert logits[0, 0] == (weight * 400) // 4, (code, weight)


def test_bit_order_lsb_first_one_hot_probes():
    # code 3 (weight +1) at slot p, code 2 (weight 0) elsewhere: only input p passes
    for p in range(4):
        byte = 0
        for s in range(4):
            byte |= (3 if s == p else 2) << (2 * s)
        for q in range(4):
            x = [0, 0, 0, 0]
            x[q] = 1000
            logits, _ = _one_layer([[byte]], [x])
            assert logits[0, 0] == (250 if q == p else 0), (p, q)


def test_shift_is_floor_division_for_every_int16():
    # weight +1 on slot 0 only: the output is floor(s/4) of the int16 input s
    byte = (2 << 6) | (2 << 4) | (2 << 2) | 3
    s = np.arange(-32768, 32768, dtype=np.int64)
    x = np.zeros((s.size, 4), dtype=np.int16)
    x[:, 0] = s
    logits, _ = _one_layer([[byte]], x)
    assert np.array_equal(logits[:, 0].astype(np.int64), s // 4)


def test_relu_only_between_hidden_layers_and_commutes_with_shift():
    # layer 1: weight +1 on slot 0 (then shift, ReLU); layer 2: weight +1 on slot 0 (shift only)
    byte = (2 << 6) | (2 << 4) | (2 << 2) | 3
    l1 = np.array([[byte]] * 4, dtype=np.uint8)          # 4 identical hidden units
    l2 = np.array([[byte]], dtype=np.uint8)
    s = np.arange(-32768, 32768, 97, dtype=np.int64)
    x = np.zeros((s.size, 4), dtype=np.int16)
    x[:, 0] = s
    logits, _ = oracle.mlp_2bit([l1, l2], [4, 4, 1], x)
    relu_after = np.maximum(s // 4, 0) // 4
    relu_before = (np.maximum(s, 0) // 4) // 4
    assert np.array_equal(logits[:, 0].astype(np.int64), relu_after)
    assert np.array_equal(relu_after, relu_before)
    # the output layer keeps negative values
    logits1, _ = _one_layer([[byte]], x)
    assert (logits1[:, 0] < 0).any()


def test_exhaustive_4_to_1_layer_against_exact_integers():
    # every code byte x 32 input patterns including the int16 boundaries
    r = np.random.default_rng(11)
    pats = [[-32768, 32767, -1, 1], [32767, 32767, 32767, 32767], [-32768] * 4, [0, 0, 0, 0],
            [-5, -4, -1, 3], [127, 0, 127, 0]]
    pats += r.integers(-32768, 32768, size=(26, 4)).tolist()
    x = np.array(pats, dtype=np.int16)
    codes = np.arange(256, dtype=np.uint8).reshape(256, 1)
    logits, am = oracle.mlp_2bit([codes], [4, 256], x)
    ref_logits, ref_am = exact.mlp_2bit([codes.tolist()], [4, 256], x.tolist())
    assert np.array_equal(logits, np.array(ref_logits, dtype=np.int16))
    assert np.array_equal(am, np.array(ref_am, dtype=np.int32))


def test_wraparound_forcing_rows_match_exact_wrap_once():
    # all codes 0 (weight -2) with inputs 64..127: the layer-1 sum is far below -32768 and wraps
    dims = [256, 192, 128, 40]
    layers = [np.zeros((dims[l + 1], dims[l] // 4), dtype=np.uint8) for l in range(3)]
    x = synth.mlp2bit_inputs(batch=4, lo=64, hi=128, extra=1)
    assert (-2 * x.astype(np.int64).sum(axis=1) < -32768).all()
    logits, am = oracle.mlp_2bit(layers, dims, x)
    ref, ref_am = exact.mlp_2bit([l.tolist() for l in layers], dims, x.tolist())
    assert np.array_equal(logits, np.array(ref, dtype=np.int16))
    assert np.array_equal(am, np.array(ref_am))


@pytest.mark.parametrize("case", ["balanced", "fullrange"])
def test_random_chains_against_exact_integers(case):
    dims = list(synth.MLP_DIMS)
    layers = synth.mlp2bit_layers(extra=5)
    if case == "balanced":
        # codes uniform on {1,2,3}: mean weight 0, so hidden units are often positive
        r = np.random.default_rng(12)
        layers = [_codes_from_values(r.integers(1, 4, size=(l.shape[0], l.shape[1] * 4)))
                  for l in layers]
        x = synth.mlp2bit_inputs(batch=6, extra=2)
    else:
        x = synth.mlp2bit_inputs(batch=6, lo=-32768, hi=32768, extra=3)
    logits, am = oracle.mlp_2bit(layers, dims, x)
    ref, ref_am = exact.mlp_2bit([l.tolist() for l in layers], dims, x.tolist())
    assert np.array_equal(logits, np.array(ref, dtype=np.int16))
    assert np.array_equal(am, np.array(ref_am))
    if case == "balanced":
        assert len(set(am.tolist())) > 1 or np.any(logits != 0)


def _codes_from_values(c):
    """uint8 [n][k/4] canonical bytes from per-weight codes [n][k] (slot j%4 at bits 2*(j%4))."""
    c = np.asarray(c, dtype=np.uint8)
    n, k = c.shape
    c4 = c.reshape(n, k // 4, 4)
    return (c4[..., 0] | (c4[..., 1] << 2) | (c4[..., 2] << 4) | (c4[..., 3] << 6)).astype(np.uint8)


def test_literal_workload_is_degenerate_all_zero_logits():
    dims = list(synth.MLP_DIMS)
    layers = synth.mlp2bit_layers()
    x = synth.mlp2bit_inputs()
    logits, am = oracle.mlp_2bit(layers, dims, x)
    assert logits.shape == (1024, 40)
    assert not logits.any()
    assert not am.any()


def test_argmax_ties_pick_lowest_index():
    # two output units with identical rows give identical logits: argmax must be 0, then 1
    byte = (2 << 6) | (2 << 4) | (2 << 2) | 3
    zero = (2 << 6) | (2 << 4) | (2 << 2) | 2
    logits, am = _one_layer([[byte], [byte], [zero]], [[400, 0, 0, 0], [-400, 0, 0, 0]])
    assert logits.tolist() == [[100, 100, 0], [-100, -100, 0]]
    assert am.tolist() == [0, 2]


def test_mac_count_order_of_magnitude():
    g = read_kv("z80_mlp_shape.txt")
    dims = [int(g["inputs"][0])] + [int(v) for v in g["hidden"]] + [40]
    assert int(g["query_buckets"][0]) + int(g["context_buckets"][0]) == dims[0]
    macs = sum(dims[i] * dims[i + 1] for i in range(len(dims) - 1))
    assert macs == 78848
    order = int(g["macs_per_char_order"][0])
    assert order / 10 ** 0.5 < macs < order * 10 ** 0.5
