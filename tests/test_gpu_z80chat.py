"""GPU parity of the Z80-uLM character loop: lbq_z80_encode bit-exact to the oracle's trigram
buckets, and lbq_z80_chat_2bit (the whole generation loop in one launch) bit-exact to the
oracle's replies and lengths, on random and hand-built weights."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from packed_weight_gemv_amd import synth
from tests._gpu import to_dev
from tests.test_oracle_z80chat import _layers_from_codes

pytestmark = pytest.mark.gpu
DIMS = list(synth.MLP_DIMS)


def _texts(texts):
    stride = max(1, max(len(t) for t in texts))
    arr = np.zeros((len(texts), stride), dtype=np.uint8)
    lens = np.zeros(len(texts), dtype=np.int32)
    for b, t in enumerate(texts):
        arr[b, :len(t)] = np.frombuffer(t, dtype=np.uint8)
        lens[b] = len(t)
    return arr, lens


def _encode(lbq, arr, lens):
    out = torch.empty((arr.shape[0], 128), dtype=torch.int16, device="cuda:0")
    lbq.lbq_z80_encode(to_dev(arr), to_dev(lens), out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _chat(lbq, layers, arr, lens, max_reply):
    lw = [to_dev(lbq.lbq_pack_2bit(c)) for c in layers]
    reply = torch.full((arr.shape[0], max_reply), 0x55, dtype=torch.uint8, device="cuda:0")
    rl = torch.full((arr.shape[0],), -7, dtype=torch.int32, device="cuda:0")
    lbq.lbq_z80_chat_2bit(lw, DIMS, to_dev(arr), to_dev(lens), reply, rl)
    torch.cuda.synchronize()
    return reply.cpu().numpy(), rl.cpu().numpy()


def _oracle_chat(layers, arr, lens, max_reply):
    prompts = [bytes(arr[b, :lens[b]]) for b in range(arr.shape[0])]
    return oracle.z80_chat(layers, DIMS, prompts, max_reply)


def test_encoder_is_bit_exact(lbq):
    arr, lens = synth.chat_prompts(257, extra=1)
    special = [b"", b"hello there", b"there hello", b"a " * 1500, b"...,,,!!??", b"Z80 uLM 4MHz",
               bytes(range(256))]
    arr2, lens2 = _texts(special)
    for a, l in ((arr, lens), (arr2, lens2)):
        got = _encode(lbq, a, l)
        want = np.stack([oracle.z80_encode(bytes(a[b, :l[b]])) for b in range(a.shape[0])])
        assert np.array_equal(got, want)


def test_encoder_clamps_lengths(lbq):
    arr, _ = _texts([b"hello there", b"abc"])
    lens = np.array([1000, -5], dtype=np.int32)
    got = _encode(lbq, arr, lens)
    assert np.array_equal(got[0], oracle.z80_encode(bytes(arr[0])))
    assert not got[1].any()


@pytest.mark.parametrize("batch,max_reply,extra", [(1, 32, 0), (5, 16, 1), (257, 32, 2),
                                                   (64, 1, 3), (9, 200, 4)])
def test_chat_is_bit_exact_on_random_weights(lbq, batch, max_reply, extra):
    layers = synth.mlp2bit_layers(extra=extra)
    arr, lens = synth.chat_prompts(batch, extra=10 + extra)
    print(f"z80 chat B={batch} max_reply={max_reply}", flush=True)
    reply, rl = _chat(lbq, layers, arr, lens, max_reply)
    _, want, wl = _oracle_chat(layers, arr, lens, max_reply)
    assert np.array_equal(rl, wl)
    assert np.array_equal(reply, want)


def test_chat_full_workload_is_bit_exact(lbq):
    layers = synth.mlp2bit_layers()
    arr, lens = synth.chat_prompts(synth.MLP_BATCH)
    reply, rl = _chat(lbq, layers, arr, lens, synth.Z80_REPLY)
    _, want, wl = _oracle_chat(layers, arr, lens, synth.Z80_REPLY)
    assert np.array_equal(rl, wl) and np.array_equal(reply, want)
    # the workload is not degenerate: replies of many lengths
    assert len(np.unique(rl)) > 5


def test_hand_built_weights(lbq):
    c1 = np.full((192, 256), 3)
    c2 = np.full((128, 192), 2); c2[:, 0] = 3
    c3 = np.full((40, 128), 2); c3[10, 0] = 3
    arr, lens = _texts([b"hi", b"hello there"])
    reply, rl = _chat(lbq, _layers_from_codes([c1, c2, c3]), arr, lens, 256)
    assert list(rl) == [256, 256] and np.all(reply == ord("I"))
    c1 = np.full((192, 256), 2); c1[0, :128] = 3; c1[1, 128:] = 3
    c2 = np.full((128, 192), 2); c2[0, 0] = 3; c2[1:5, 1] = 3
    c3 = np.full((40, 128), 2); c3[5, 0] = 3; c3[0, 1:5] = 3
    reply, rl = _chat(lbq, _layers_from_codes([c1, c2, c3]), *_texts([b"hi"]), 10)
    assert list(rl) == [1] and bytes(reply[0]) == b"D" + b"\0" * 9
    zero = _layers_from_codes([np.full((DIMS[i + 1], DIMS[i]), 2) for i in range(3)])
    reply, rl = _chat(lbq, zero, *_texts([b"hello", b""]), 8)
    assert not rl.any() and not reply.any()


def test_zero_reply_cap_and_rejected_shapes(lbq):
    layers = synth.mlp2bit_layers()
    arr, lens = synth.chat_prompts(3)
    reply, rl = _chat(lbq, layers, arr, lens, 0)
    assert not rl.any()
    lib = lbq.load()
    lw = [to_dev(lbq.lbq_pack_2bit(c)) for c in layers]
    ptrs = (ctypes.c_void_p * 3)(*[w.data_ptr() for w in lw])
    pr, ln = to_dev(arr), to_dev(lens)
    out = torch.zeros((3, 8), dtype=torch.uint8, device="cuda:0")
    ol = torch.full((3,), 9, dtype=torch.int32, device="cuda:0")

    def call(dims, max_reply=8):
        d = (ctypes.c_int32 * 4)(*dims)
        return lib.lbq_z80_chat_2bit(ctypes.cast(ptrs, ctypes.c_void_p), ctypes.cast(d, ctypes.c_void_p),
                                     3, ctypes.c_void_p(pr.data_ptr()), ctypes.c_void_p(ln.data_ptr()),
                                     arr.shape[1], 3, max_reply, ctypes.c_void_p(out.data_ptr()),
                                     ctypes.c_void_p(ol.data_ptr()), None)

    assert call([128, 192, 128, 40]) == -2        # input must be 128 + 128 buckets
    assert call([256, 192, 128, 41]) == -2        # outputs must be the 40-symbol charset
    assert call([256, 1008, 1008, 40]) == -4      # codes beyond the 48 KiB LDS budget
    assert call(DIMS, 257) == -2                  # reply cap
    torch.cuda.synchronize()
    assert bool((ol == 9).all()) and not bool(out.any())
