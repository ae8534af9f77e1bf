"""Entry points running concurrently on two streams (and from two host threads) must give the
results each gives alone: the library's workspaces (split-K partials and counters, the decode
step's stage workspace) are kept per stream, so concurrent work never shares them."""
import threading

import numpy as np
import pytest
import torch

from packed_weight_gemv_amd import synth
from tests._gpu import bits, empty_bf16, to_dev

pytestmark = pytest.mark.gpu

L, HID, KV, FFN = 2, 1024, 256, 2048


def _stream_work(lbq, tag):
    """The work one stream runs: a batch-1 decode step (stage kernels), a batch-2 decode step
    (per-projection GEMMs and rescales), split-K batch-1 Q1 and INT4 GEMVs (k = 16384) and a
    batch-4 Q1 GEMM. Returns (run, outputs)."""
    layers = [{nm: to_dev(lbq.lbq_pack_q1g128(*(lambda mm: (mm.signs, mm.scales))(
        synth.stream_matrix(l + 2 * tag, nm, hidden=HID, kv=KV, ffn=FFN))))
        for nm in synth.STREAM_MATRICES} for l in range(L)]
    arr = lbq.make_layers(layers)
    x1 = to_dev(synth.activations(1, HID, workload=90 + tag))
    x2 = to_dev(synth.activations(2, HID, workload=92 + tag))
    act1 = torch.zeros(lbq.lbq_decode_act_elems(L, HID, KV, FFN, 1), dtype=torch.int16,
                       device="cuda:0")
    act2 = torch.zeros(lbq.lbq_decode_act_elems(L, HID, KV, FFN, 2), dtype=torch.int16,
                       device="cuda:0")
    n, k = 320, 16384
    mq = synth.q1_matrix(n, k, workload=94, matrix=tag)
    wq = to_dev(lbq.lbq_pack_q1g128(mq.signs, mq.scales))
    mi = synth.i4_matrix(n, k, workload=95 + tag)
    wi = to_dev(lbq.lbq_pack_i4g128(mi.nib, mi.scales))
    xk1 = to_dev(synth.activations(1, k, workload=96 + tag))
    xk4 = to_dev(synth.activations(4, k, workload=98 + tag))
    yq, yi, yg = empty_bf16(1, n), empty_bf16(1, n), empty_bf16(4, n)

    def run(stream):
        lbq.lbq_decode_step_q1g128(arr, L, HID, KV, FFN, x1, act1, stream=stream)
        lbq.lbq_gemv_q1g128(wq, n, k, xk1, yq, stream=stream)
        lbq.lbq_decode_step_q1g128(arr, L, HID, KV, FFN, x2, act2, stream=stream)
        lbq.lbq_gemv_i4g128(wi, n, k, xk1, yi, stream=stream)
        lbq.lbq_gemv_q1g128(wq, n, k, xk4, yg, stream=stream)

    return run, [act1, act2, yq, yi, yg]


def _snapshot(outs):
    torch.cuda.synchronize()
    return [bits(o).copy() for o in outs]


def _clear(outs):
    for o in outs:
        o.fill_(0x7FC0)   # bf16 NaN: a slot left unwritten cannot match
    torch.cuda.synchronize()


@pytest.mark.parametrize("threads", [False, True])
def test_two_streams_match_serial(lbq, threads):
    work = [_stream_work(lbq, t) for t in range(2)]
    streams = [torch.cuda.Stream() for _ in range(2)]
    torch.cuda.synchronize()   # the uploads (on the default stream) are complete
    serial = []
    for (run, outs), s in zip(work, streams):
        run(s)   # alone: nothing else is queued
        serial.append(_snapshot(outs))
    for rep in range(3):
        for _, outs in work:
            _clear(outs)
        if threads:
            ts = [threading.Thread(target=lambda r=run, s=s: [r(s) for _ in range(2)])
                  for (run, _), s in zip(work, streams)]
            for t in ts:
                t.start()
            for t in ts:
                t.join()
        else:
            for _ in range(2):
                for (run, _), s in zip(work, streams):
                    run(s)
        for (_, outs), ref in zip(work, serial):
            got = _snapshot(outs)
            for g, r in zip(got, ref):
                assert np.array_equal(g, r)
