"""GPU parity of the RMS rescale and of the Q1_0_g128 decode step: every GEMV of the step is
checked with teacher forcing (the oracle evaluates it on the GPU's own bf16 input), every
rescale to within one bf16 ulp of the oracle."""
import numpy as np
import pytest
import torch

import oracle
from packed_weight_gemv_amd import synth
from tests._gpu import bf16_ordinal, bits, check_within, empty_bf16, to_dev

pytestmark = pytest.mark.gpu


def _check_rms(y_bits, x_bits, y2_bits=None, eps=1e-6):
    ref, exact_q = oracle.rms_rescale(y_bits, y2_bits, eps)
    d = np.abs(bf16_ordinal(x_bits) - bf16_ordinal(ref))
    assert d.max() <= 1, f"rescale differs by {d.max()} ulp"
    return int((d == 1).sum())


@pytest.mark.parametrize("n,batch,prod", [(5120, 1, False), (17408, 8, True), (300, 3, False),
                                          (1, 2, False)])
def test_rms_rescale_within_one_ulp(lbq, n, batch, prod):
    y = synth.activations(batch, n, workload=50, extra=n)
    y2 = synth.activations(batch, n, workload=51, extra=n) if prod else None
    x = empty_bf16(batch, n)
    lbq.lbq_rms_rescale_bf16(to_dev(y), x, to_dev(y2) if prod else None, eps=1e-6)
    torch.cuda.synchronize()
    ones = _check_rms(y, bits(x), y2)
    assert ones <= max(2, n * batch // 1000)


def _build_stream(lbq, L, hid, kv, ffn):
    mats, layers = [], []
    for l in range(L):
        d = {name: synth.stream_matrix(l, name, hid, kv, ffn) for name in synth.STREAM_MATRICES}
        mats.append(d)
        layers.append({nm: to_dev(lbq.lbq_pack_q1g128(m.signs, m.scales)) for nm, m in d.items()})
    return mats, layers


def _check_step(lbq, mats, act, L, hid, kv, ffn, batch, layers_to_check, rows=None):
    view = lambda s, l: bits(lbq.act_view(act, s, l, L, hid, kv, ffn, batch))
    for l in layers_to_check:
        for name, src in (("q", "x"), ("k", "x"), ("v", "x"), ("gate", "x"), ("up", "x"),
                          ("o", "xo"), ("down", "xd")):
            m = mats[l][name]
            n = m.shape[0]
            r = None if rows is None else np.unique(np.concatenate(
                [np.arange(0, n, max(1, n // rows)), [n - 1]])).astype(np.int32)
            ref, l1 = oracle.gemv_q1g128(m.signs, m.scales, view(src, l), rows=r)
            y = view(name, l)
            check_within(y if r is None else y[:, r], ref, l1, f"layer {l} {name}")
        _check_rms(view("q", l), view("xo", l))
        _check_rms(view("gate", l), view("xd", l), view("up", l))
        nxt = view("x", l + 1) if l + 1 < L else view("final", L)
        _check_rms(view("down", l), nxt)


@pytest.mark.parametrize("batch", [1, 2, 5, 8, 16])
def test_decode_step_small_stream_teacher_forced(lbq, batch):
    L, hid, kv, ffn = 3, 384, 128, 640
    mats, layers = _build_stream(lbq, L, hid, kv, ffn)
    arr = lbq.make_layers(layers)
    x0 = synth.activations(batch, hid, workload=synth.W_Q1_STREAM, extra=batch)
    act = torch.zeros(lbq.lbq_decode_act_elems(L, hid, kv, ffn, batch), dtype=torch.int16,
                      device="cuda:0")
    lbq.lbq_decode_step_q1g128(arr, L, hid, kv, ffn, to_dev(x0), act)
    torch.cuda.synchronize()
    assert np.array_equal(bits(lbq.act_view(act, "x", 0, L, hid, kv, ffn, batch)), x0)
    _check_step(lbq, mats, act, L, hid, kv, ffn, batch, range(L))


@pytest.mark.parametrize("batch", [1, 8])
def test_decode_step_27b_shapes_two_layers_sampled(lbq, batch):
    L, hid, kv, ffn = 2, synth.STREAM_HIDDEN, synth.STREAM_KV, synth.STREAM_FFN
    mats, layers = _build_stream(lbq, L, hid, kv, ffn)
    arr = lbq.make_layers(layers)
    x0 = synth.activations(batch, hid, workload=synth.W_Q1_STREAM, extra=batch - 1)
    act = torch.zeros(lbq.lbq_decode_act_elems(L, hid, kv, ffn, batch), dtype=torch.int16,
                      device="cuda:0")
    lbq.lbq_decode_step_q1g128(arr, L, hid, kv, ffn, to_dev(x0), act)
    torch.cuda.synchronize()
    _check_step(lbq, mats, act, L, hid, kv, ffn, batch, range(L), rows=61)


def test_decode_step_unaligned_input(lbq):
    """A step input 4-byte but not 16-byte aligned is refused by the stage kernels (their LDS
    copies need 16 bytes) and served by another path, still in teacher-forced parity; one that
    is not 4-byte aligned is rejected with LBQ_E_ALIGN and leaves the record untouched."""
    L, hid, kv, ffn, batch = 2, 384, 128, 640, 1
    mats, layers = _build_stream(lbq, L, hid, kv, ffn)
    arr = lbq.make_layers(layers)
    x0 = synth.activations(batch, hid, workload=synth.W_Q1_STREAM, extra=7)
    buf = torch.zeros(hid + 8, dtype=torch.int16, device="cuda:0")
    n = lbq.lbq_decode_act_elems(L, hid, kv, ffn, batch)
    act = torch.zeros(n, dtype=torch.int16, device="cuda:0")
    odd = buf[1:1 + hid].view(batch, hid)      # 2 bytes past a 256-byte aligned allocation
    odd.copy_(to_dev(x0))
    with pytest.raises(lbq.LbqError, match="LBQ_E_ALIGN"):
        lbq.lbq_decode_step_q1g128(arr, L, hid, kv, ffn, odd, act)
    torch.cuda.synchronize()
    assert not act.any()
    view = buf[2:2 + hid].view(batch, hid)     # 4 bytes past it
    view.copy_(to_dev(x0))
    assert view.data_ptr() % 16 == 4
    lbq.lbq_decode_step_q1g128(arr, L, hid, kv, ffn, view, act)
    torch.cuda.synchronize()
    assert np.array_equal(bits(lbq.act_view(act, "x", 0, L, hid, kv, ffn, batch)), x0)
    _check_step(lbq, mats, act, L, hid, kv, ffn, batch, range(L))
