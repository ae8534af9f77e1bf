"""Pins of the oracle's Z80-uLM character loop: the trigram hash (FNV-1a, pinned by its published
test vectors), the trigram encoder (the page's word-order invariance and typo tolerance, one
trigram per letter, steps of 32, saturation), and the generation loop (constructed weights whose
replies follow by hand, and step-by-step agreement with the exact Python MLP twin)."""
import os

import numpy as np
import pytest

import oracle
from oracle import exact

GOLD = os.path.join(os.path.dirname(__file__), "golden")
DIMS = [256, 192, 128, 40]


def _gold(name):
    with open(os.path.join(GOLD, name)) as fh:
        return [l.rstrip("\n") for l in fh if l.strip() and not l.startswith("#")]


def test_fnv1a32_published_vectors():
    for line in _gold("fnv1a32_vectors.txt"):
        text, hx = line.rsplit(" ", 1)
        assert oracle.fnv1a32(text.strip('"').encode()) == int(hx, 16), line


def test_normalization_keeps_the_charset_and_spaces_the_rest():
    kept = 0
    for c in range(256):
        v = oracle.z80_normalize(c)
        ch = chr(c)
        if "a" <= ch <= "z":
            assert v == ord(ch.upper())
        elif ch.isascii() and (ch.isupper() or ch.isdigit() or ch in "?!"):
            assert v == c
        else:
            assert v == ord(" ")
        kept += v != ord(" ")
    assert kept == 26 * 2 + 10 + 2
    assert len(oracle.Z80_CHARSET) == 40


def test_page_example_order_invariance_and_typo_tolerance():
    rows = [l.split(" | ") for l in _gold("z80_encoder_example.txt")]
    for a, b, rel in rows:
        ea, eb = oracle.z80_encode(a.encode()), oracle.z80_encode(b.encode())
        if rel == "equal":
            assert np.array_equal(ea, eb)
        else:
            shared = int(np.minimum(ea, eb).sum()) // 32
            # "helo" keeps " HE", "HEL", "LO "; "ther" keeps " TH", "THE", "HER"
            assert shared >= 6 and not np.array_equal(ea, eb)


@pytest.mark.parametrize("text", [b"hello there", b"a", b"Are you a ROBOT?", b"x  y   z9!", b"",
                                  b"...,,,"])
def test_one_trigram_per_letter_in_steps_of_32(text):
    e = oracle.z80_encode(text)
    letters = sum(oracle.z80_normalize(c) != ord(" ") for c in text)
    assert np.all(e % 32 == 0) and np.all(e >= 0)
    assert int(e.sum()) == 32 * letters


def test_single_letter_lands_in_its_padded_trigram_bucket():
    e = oracle.z80_encode(b"a")
    idx = oracle.fnv1a32(b" A ") % 128
    assert e[idx] == 32 and int(e.sum()) == 32


def test_punctuation_and_case_do_not_matter():
    assert np.array_equal(oracle.z80_encode(b"Hello, there."), oracle.z80_encode(b"HELLO THERE"))


def test_buckets_saturate_at_int16_max():
    e = oracle.z80_encode(b"a " * 1100)
    assert e[oracle.fnv1a32(b" A ") % 128] == 32767


def _layers_from_codes(codes_list):
    """Canonical packed layers from full code matrices (code c of input j in bits 2(j%4))."""
    out = []
    for c in codes_list:
        n, k = c.shape
        q = c.reshape(n, k // 4, 4).astype(np.uint8)
        out.append((q[:, :, 0] | (q[:, :, 1] << 2) | (q[:, :, 2] << 4) | (q[:, :, 3] << 6)).astype(np.uint8))
    return out


def test_zero_weights_end_every_reply_at_once():
    layers = _layers_from_codes([np.full((DIMS[i + 1], DIMS[i]), 2) for i in range(3)])
    replies, rep, rl = oracle.z80_chat(layers, DIMS, [b"hello", b"", b"are you a bot"], 16)
    assert replies == [b"", b"", b""] and not rep.any() and not rl.any()


def test_a_constant_winner_fills_the_reply():
    # L1 all +1 (h1 = floor(sum a / 4)), L2 row r: +1 on h1[0] only, L3 row 10 ('I'): +1 on
    # h2[0] only, everything else 0. With a prompt of two letters, sum a >= 64, so logit 10 >= 1
    # and every other logit is 0: the reply is 'I' repeated up to the cap.
    c1 = np.full((192, 256), 3)
    c2 = np.full((128, 192), 2); c2[:, 0] = 3
    c3 = np.full((40, 128), 2); c3[10, 0] = 3
    layers = _layers_from_codes([c1, c2, c3])
    replies, _, rl = oracle.z80_chat(layers, DIMS, [b"hi", b"hello there"], 12)
    assert replies == [b"I" * 12, b"I" * 12] and list(rl) == [12, 12]


def test_the_context_buckets_can_stop_the_reply():
    # query path: h1[0] = floor(sum query / 4) -> h2[0] = floor(h1[0] / 4) -> logit 5 ('D')
    # context path: h1[1] = floor(sum context / 4) -> h2[1..4] = floor(h1[1] / 4) -> logit 0
    # (end) = floor(sum of the four / 4). Prompt "hi": sum query = 64, h1[0] = 16, h2[0] = 4,
    # logit 5 = 1. Before any output the context is empty (logit 0 = 0): 'D' is emitted. After
    # it the context holds one trigram (32): h1[1] = 8, h2[1..4] = 2, logit 0 = 2 > 1: stop.
    c1 = np.full((192, 256), 2); c1[0, :128] = 3; c1[1, 128:] = 3
    c2 = np.full((128, 192), 2); c2[0, 0] = 3; c2[1:5, 1] = 3
    c3 = np.full((40, 128), 2); c3[5, 0] = 3; c3[0, 1:5] = 3
    layers = _layers_from_codes([c1, c2, c3])
    replies, _, rl = oracle.z80_chat(layers, DIMS, [b"hi"], 10)
    assert replies == [b"D"] and list(rl) == [1]


def test_every_step_is_the_argmax_of_the_exact_mlp_twin():
    r = np.random.default_rng(77)
    codes = [r.integers(0, 4, size=(DIMS[i + 1], DIMS[i])) for i in range(3)]
    # bias the last layer's code distribution so that replies run for a few characters
    layers = _layers_from_codes(codes)
    prompts = [b"hello", b"are you a robot", b"do you dream", b"zx 81", b"?"]
    replies, _, rl = oracle.z80_chat(layers, DIMS, prompts, 8)
    for p, rep, n in zip(prompts, replies, rl):
        q = oracle.z80_encode(p)
        for t in range(n + 1):
            if t == 8:
                break
            x = np.concatenate([q, oracle.z80_encode(rep[:t])]).astype(np.int16)[None, :]
            _, am = exact.mlp_2bit(layers, DIMS, x)
            want = 0 if t == n else oracle.Z80_CHARSET.index(rep[t])
            assert int(am[0]) == want, (p, t)
