"""Seeded synthetic inputs in the canonical layouts, shared by the tests, the bench and the
smoke check. This module draws random numbers and stores them in the documented canonical
layouts; it performs none of the method's arithmetic and imports neither the library nor the
oracle.

Seeds: numpy PCG64 seeded with [0x1B0, workload, layer, matrix, kind, extra], kind 0 = codes /
sign bits, 1 = scales, 2 = activations / inputs, 3 = stress patterns.

Distributions (per workload):
  * sign bits, int4 nibbles, 2-bit codes: uniform random bytes, i.e. iid Bernoulli(0.5) sign
    bits, uniform -8..7 nibbles and uniform 0..3 codes;
  * scales: fp16(|N(0, sigma)|), round to nearest even, sigma 0.02 (Q1) or 0.01 (INT4);
  * activations: bf16(N(0, 1)), drawn as float32 and rounded to nearest even;
  * 2-bit MLP inputs: int16 uniform on 0..127 (128 query + 128 context bucket counts).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SEED_ROOT = 0x1B0
KIND_CODES, KIND_SCALES, KIND_ACT, KIND_STRESS = 0, 1, 2, 3

# workload ids
W_MLP2BIT, W_Q1_SQUARE, W_Q1_MLP, W_I4_LAYER, W_Q1_STREAM = 1, 2, 3, 4, 5
W_Z80_CHAT = 6
W_TERN = 7
Z80_REPLY = 32                          # reply cap of the chat-loop workload

MLP_DIMS = (256, 192, 128, 40)          # 128 query + 128 context buckets -> ... -> 40 chars
MLP_BATCH = 1024
Q1_SIGMA = 0.02
I4_SIGMA = 0.01

# 27B-shaped stream: 64 layers of q, k, v, o, gate, up, down
STREAM_LAYERS = 64
STREAM_HIDDEN = 5120
STREAM_KV = 1024
STREAM_FFN = 17408
STREAM_MATRICES = ("q", "k", "v", "o", "gate", "up", "down")

# Qwen3-8B-shaped INT4 layer: (name, n, k)
I4_SHAPES = (("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
             ("gate", 12288, 4096), ("up", 12288, 4096), ("down", 4096, 12288))


def rng(workload: int, layer: int = 0, matrix: int = 0, kind: int = 0, extra: int = 0):
    return np.random.default_rng([SEED_ROOT, workload, layer, matrix, kind, extra])


def random_bytes(r: np.random.Generator, shape) -> np.ndarray:
    count = int(np.prod(shape))
    return np.frombuffer(r.bytes(count), dtype=np.uint8).reshape(shape).copy()


def fp16_abs_normal(r: np.random.Generator, shape, sigma: float) -> np.ndarray:
    """fp16 bit patterns of |N(0, sigma)|, drawn in float32 (numpy's float32 -> float16 cast
    rounds to nearest even and keeps subnormals)."""
    z = r.standard_normal(size=shape, dtype=np.float32)
    return np.abs(z * np.float32(sigma)).astype(np.float16).view(np.uint16)


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_normal(r: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(r.standard_normal(size=shape, dtype=np.float32))


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (a reinterpretation)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


@dataclass
class Q1Matrix:
    signs: np.ndarray   # uint8 [n][k/8]
    scales: np.ndarray  # fp16 bits [n][k/128]

    @property
    def shape(self):
        return self.signs.shape[0], self.signs.shape[1] * 8


@dataclass
class I4Matrix:
    nib: np.ndarray     # uint8 [n][k/2]
    scales: np.ndarray  # fp16 bits [n][k/128]

    @property
    def shape(self):
        return self.nib.shape[0], self.nib.shape[1] * 2


def q1_matrix(n: int, k: int, workload: int, layer: int = 0, matrix: int = 0,
              sigma: float = Q1_SIGMA) -> Q1Matrix:
    signs = random_bytes(rng(workload, layer, matrix, KIND_CODES), (n, k // 8))
    scales = fp16_abs_normal(rng(workload, layer, matrix, KIND_SCALES), (n, k // 128), sigma)
    return Q1Matrix(signs, scales)


def i4_matrix(n: int, k: int, workload: int, layer: int = 0, matrix: int = 0,
              sigma: float = I4_SIGMA) -> I4Matrix:
    nib = random_bytes(rng(workload, layer, matrix, KIND_CODES), (n, k // 2))
    scales = fp16_abs_normal(rng(workload, layer, matrix, KIND_SCALES), (n, k // 128), sigma)
    return I4Matrix(nib, scales)


@dataclass
class TernMatrix:
    codes: np.ndarray    # uint8 [n][k] in {0, 1, 2}, weight = code - 1
    scales: np.ndarray   # fp16 bits [n][ceil(k/160)]

    @property
    def shape(self):
        return self.codes.shape


def tern_matrix(n: int, k: int, workload: int = W_TERN, layer: int = 0, matrix: int = 0,
                sigma: float = Q1_SIGMA) -> TernMatrix:
    """Ternary weights uniform over {-1, 0, +1}, fp16 scales |N(0, sigma)| per 160 weights."""
    codes = rng(workload, layer, matrix, KIND_CODES).integers(0, 3, size=(n, k), dtype=np.uint8)
    scales = fp16_abs_normal(rng(workload, layer, matrix, KIND_SCALES), (n, (k + 159) // 160), sigma)
    return TernMatrix(codes, scales)


def activations(batch: int, k: int, workload: int, layer: int = 0, matrix: int = 0,
                extra: int = 0) -> np.ndarray:
    return bf16_normal(rng(workload, layer, matrix, KIND_ACT, extra), (batch, k))


def mlp2bit_layers(dims=MLP_DIMS, workload: int = W_MLP2BIT, extra: int = 0):
    """Canonical 2-bit codes per layer: uint8 [dims[l+1]][dims[l]/4], uniform bytes."""
    return [random_bytes(rng(workload, l, 0, KIND_CODES, extra), (dims[l + 1], dims[l] // 4))
            for l in range(len(dims) - 1)]


def mlp2bit_inputs(batch: int = MLP_BATCH, width: int = MLP_DIMS[0], workload: int = W_MLP2BIT,
                   lo: int = 0, hi: int = 128, extra: int = 0) -> np.ndarray:
    r = rng(workload, 0, 0, KIND_ACT, extra)
    return r.integers(lo, hi, size=(batch, width), dtype=np.int64).astype(np.int16)


def stream_shape(name: str, hidden=STREAM_HIDDEN, kv=STREAM_KV, ffn=STREAM_FFN):
    """(n, k) of a projection of the 27B-shaped stream."""
    return {"q": (hidden, hidden), "k": (kv, hidden), "v": (kv, hidden), "o": (hidden, hidden),
            "gate": (ffn, hidden), "up": (ffn, hidden), "down": (hidden, ffn)}[name]


def stream_matrix(layer: int, name: str, hidden=STREAM_HIDDEN, kv=STREAM_KV,
                  ffn=STREAM_FFN) -> Q1Matrix:
    n, k = stream_shape(name, hidden, kv, ffn)
    return q1_matrix(n, k, W_Q1_STREAM, layer, STREAM_MATRICES.index(name))


def stream_bytes_per_layer(hidden=STREAM_HIDDEN, kv=STREAM_KV, ffn=STREAM_FFN) -> int:
    """Algorithmic packed bytes of one layer (codes + scales, 1.125 bits per weight)."""
    total = 0
    for name in STREAM_MATRICES:
        n, k = stream_shape(name, hidden, kv, ffn)
        total += n * k * 9 // 64
    return total


def chat_prompts(batch: int, workload: int = W_Z80_CHAT, extra: int = 0, max_words: int = 5,
                 max_word: int = 8):
    """Short, varied chat inputs (the Z80-uLM page's regime: a few words): 1..max_words words of
    1..max_word characters, mostly lower-case letters with some upper case, digits and '?',
    joined by a space or ", ". Returns (uint8 [batch][stride] zero-padded, int32 lengths)."""
    r = rng(workload, 0, 0, KIND_ACT, extra)
    pool = np.frombuffer(b"abcdefghijklmnopqrstuvwxyz" * 3 + b"ABCDEFGHIJKLMNOPQRSTUVWXYZ"
                         + b"0123456789?", dtype=np.uint8)
    texts = []
    for _ in range(batch):
        words = []
        for _ in range(int(r.integers(1, max_words + 1))):
            words.append(bytes(pool[r.integers(0, pool.size, size=int(r.integers(1, max_word + 1)))]))
        sep = [b" ", b", "]
        t = words[0]
        for w in words[1:]:
            t += sep[int(r.integers(0, 2))] + w
        texts.append(t)
    stride = max(1, max(len(t) for t in texts))
    arr = np.zeros((batch, stride), dtype=np.uint8)
    lens = np.zeros(batch, dtype=np.int32)
    for b, t in enumerate(texts):
        arr[b, :len(t)] = np.frombuffer(t, dtype=np.uint8)
        lens[b] = len(t)
    return arr, lens

