"""Calls captured in a HIP graph and replayed: every replay (with eager work and synchronisation
between replays) must match the eager result. Eager and captured calls run the same kernels, so
they must agree bitwise; batch-1 Q1 GEMVs are also held to the oracle's tolerance."""
import numpy as np
import pytest
import torch

import oracle
from packed_weight_gemv_amd import synth
from tests._gpu import bits, check_within, empty_bf16, to_dev

pytestmark = pytest.mark.gpu


def _replays(graph, outs, eager_work, count=3):
    got = []
    for r in range(count):
        eager_work()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got.append([bits(o).copy() for o in outs])
    return got


def test_batch1_q1_gemvs_in_a_graph(lbq):
    shapes = [(320, 1024), (200, 2048), (64, 5120)]
    mats = [synth.q1_matrix(n, k, workload=70, matrix=i) for i, (n, k) in enumerate(shapes)]
    ws = [to_dev(lbq.lbq_pack_q1g128(m.signs, m.scales)) for m in mats]
    xs = [to_dev(synth.activations(1, k, workload=70, extra=i)) for i, (_, k) in enumerate(shapes)]
    ys = [empty_bf16(1, n) for n, _ in shapes]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):   # eager first: the split-K workspace exists before capture
        for w, (n, k), x, y in zip(ws, shapes, xs, ys):
            lbq.lbq_gemv_q1g128(w, n, k, x, y)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for w, (n, k), x, y in zip(ws, shapes, xs, ys):
            lbq.lbq_gemv_q1g128(w, n, k, x, y)
    junk = empty_bf16(1, 320)

    def eager():   # an eager call between replays, writing elsewhere
        lbq.lbq_gemv_q1g128(ws[0], 320, 1024, xs[0], junk)

    reps = _replays(g, ys, eager)
    for r in reps[1:]:
        for a, b in zip(reps[0], r):
            assert np.array_equal(a, b)
    for m, x, y in zip(mats, xs, reps[-1]):
        ref, l1 = oracle.gemv_q1g128(m.signs, m.scales, bits(x))
        check_within(y, ref, l1, "captured q1 gemv")


@pytest.mark.parametrize("path", ["i4", "i8act", "tern"])
def test_per_call_gemvs_in_a_graph_match_eager(lbq, path):
    n, k, B = 300, 4096, 1
    x = to_dev(synth.activations(B, k, workload=71))
    if path == "tern":
        m = synth.tern_matrix(n, k, matrix=71)
        w = to_dev(lbq.lbq_pack_tern_g160(m.codes, m.scales))
        fn = lbq.lbq_gemv_tern_g160
    else:
        m = synth.i4_matrix(n, k, workload=71)
        w = to_dev(lbq.lbq_pack_i4g128(m.nib, m.scales))
        fn = lbq.lbq_gemv_i4g128 if path == "i4" else lbq.lbq_gemv_i4g128_act_i8
    y_eager = empty_bf16(B, n)
    y = empty_bf16(B, n)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        fn(w, n, k, x, y_eager)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn(w, n, k, x, y)
    reps = _replays(g, [y], lambda: fn(w, n, k, x, y_eager))
    for r in reps:
        assert np.array_equal(r[0], bits(y_eager))


@pytest.mark.parametrize("batch", [1, 4])
def test_decode_step_in_a_graph_matches_eager_and_is_deterministic(lbq, batch):
    """Batch 1 runs the stage kernels, batch 4 the matrix-core GEMV launches (split-K tile
    counters re-armed by every launch) and the wide rescale launches between them."""
    L, hid, kv, ffn = 2, 1024, 256, 2048
    layers = [{nm: to_dev(lbq.lbq_pack_q1g128(*(lambda mm: (mm.signs, mm.scales))(
        synth.stream_matrix(l, nm, hidden=hid, kv=kv, ffn=ffn)))) for nm in synth.STREAM_MATRICES}
        for l in range(L)]
    arr = lbq.make_layers(layers)
    x0 = to_dev(synth.activations(batch, hid, workload=72))
    n = lbq.lbq_decode_act_elems(L, hid, kv, ffn, batch)
    act_a = torch.zeros(n, dtype=torch.int16, device="cuda:0")
    act_b = torch.zeros(n, dtype=torch.int16, device="cuda:0")
    act_g = torch.zeros(n, dtype=torch.int16, device="cuda:0")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        lbq.lbq_decode_step_q1g128(arr, L, hid, kv, ffn, x0, act_a)
        lbq.lbq_decode_step_q1g128(arr, L, hid, kv, ffn, x0, act_b)
    torch.cuda.synchronize()
    assert np.array_equal(bits(act_a), bits(act_b))   # two eager steps agree bitwise
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        lbq.lbq_decode_step_q1g128(arr, L, hid, kv, ffn, x0, act_g)
    reps = _replays(g, [act_g], lambda: lbq.lbq_decode_step_q1g128(arr, L, hid, kv, ffn, x0, act_b))
    for r in reps:
        assert np.array_equal(r[0], bits(act_a))
