"""The allocation-free batch-1 decode step (static scratch array) against the allocating entry
point: two calls in a row, the second with a smaller input, each bitwise equal to
lbq_decode_step_q1g128 on the same inputs."""
import numpy as np
import pytest
import torch

from packed_weight_gemv_amd import synth
from tests._gpu import bits, to_dev

pytestmark = pytest.mark.gpu


def _case(lbq, L, hid, kv, ffn, workload):
    layers = [{nm: to_dev(lbq.lbq_pack_q1g128(*(lambda mm: (mm.signs, mm.scales))(
        synth.stream_matrix(l, nm, hidden=hid, kv=kv, ffn=ffn)))) for nm in synth.STREAM_MATRICES}
        for l in range(L)]
    arr = lbq.make_layers(layers)
    x0 = to_dev(synth.activations(1, hid, workload=workload))
    n = lbq.lbq_decode_act_elems(L, hid, kv, ffn, 1)
    ref = torch.zeros(n, dtype=torch.int16, device="cuda:0")
    got = torch.full((n,), 0x7FC0, dtype=torch.int16, device="cuda:0")   # bf16 NaN everywhere
    torch.cuda.synchronize()
    return arr, x0, ref, got


def test_noalloc_decode_step_matches_the_allocating_step(lbq):
    cases = [(2, synth.STREAM_HIDDEN, synth.STREAM_KV, synth.STREAM_FFN, 60),   # 27B shapes
             (1, 1024, 256, 2048, 61)]                                           # then smaller
    for L, hid, kv, ffn, wl in cases:
        arr, x0, ref, got = _case(lbq, L, hid, kv, ffn, wl)
        lbq.lbq_decode_step_q1g128_noalloc(arr, L, hid, kv, ffn, x0, got)
        lbq.lbq_decode_step_q1g128(arr, L, hid, kv, ffn, x0, ref)
        torch.cuda.synchronize()
        g, r = bits(got), bits(ref)
        assert np.array_equal(g, r), f"{L} layers, hidden {hid}: {np.count_nonzero(g != r)} differ"


def test_noalloc_decode_step_rejects_what_it_cannot_serve(lbq):
    L, hid, kv, ffn = 1, 1024, 256, 2048
    arr, x0, ref, got = _case(lbq, L, hid, kv, ffn, 62)
    x2 = to_dev(synth.activations(2, hid, workload=63))
    act2 = torch.zeros(lbq.lbq_decode_act_elems(L, hid, kv, ffn, 2), dtype=torch.int16,
                       device="cuda:0")
    with pytest.raises(lbq.LbqError, match="LBQ_E_UNSUPPORTED"):
        lbq.lbq_decode_step_q1g128_noalloc(arr, L, hid, kv, ffn, x2, act2)   # batch 2
    torch.cuda.synchronize()
    assert not act2.any()
