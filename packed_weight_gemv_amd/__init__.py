"""packed_weight_gemv_amd - Python binding of liblbq.so, the packed low-bit GEMV library for
AMD MI355X (gfx950).

The functions below carry the names of the C ABI (include/lbq.h) and only marshal arguments:
torch tensors supply device memory (`data_ptr()`) and the current HIP stream; every step of the
computation runs in the library's HIP kernels. There is no CPU fallback: if liblbq.so is not
built or cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "liblbq.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "lbq.h")

LBQ_OK = 0
STATUS = {0: "LBQ_OK", -1: "LBQ_E_NULL", -2: "LBQ_E_SHAPE", -3: "LBQ_E_ALIGN",
          -4: "LBQ_E_UNSUPPORTED", -5: "LBQ_E_ALIAS", -6: "LBQ_E_DEVICE", -7: "LBQ_E_NOMEM",
          -8: "LBQ_E_VALUE"}
MAX_BATCH = 16
Z80_MAX_REPLY = 256
ACT_SLOTS = ("x", "q", "k", "v", "gate", "up", "xo", "o", "xd", "down")

_lib = None


class LbqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")


class Q1Layer(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in ("q", "k", "v", "o", "gate", "up", "down")]


def load():
    """Loads liblbq.so (raises if it is missing: build it with __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "lbq_abi_version": ([], i32),
        "lbq_status_string": ([i32], ctypes.c_char_p),
        "lbq_2bit_bytes": ([i32, i32], sz),
        "lbq_pack_2bit": ([P, i32, i32, P], i32),
        "lbq_unpack_2bit": ([P, i32, i32, P], i32),
        "lbq_mlp_2bit_i16": ([P, P, i32, P, P, P, i32, P], i32),
        "lbq_q1g128_bytes": ([i32, i32], sz),
        "lbq_pack_q1g128": ([P, P, i32, i32, P], i32),
        "lbq_unpack_q1g128": ([P, i32, i32, P, P], i32),
        "lbq_gemv_q1g128": ([P, i32, i32, P, P, i32, P], i32),
        "lbq_i4g128_bytes": ([i32, i32], sz),
        "lbq_pack_i4g128": ([P, P, i32, i32, P], i32),
        "lbq_unpack_i4g128": ([P, i32, i32, P, P], i32),
        "lbq_gemv_i4g128": ([P, i32, i32, P, P, i32, P], i32),
        "lbq_gemm_q1g128": ([P, i32, i32, P, P, i32, P], i32),
        "lbq_gemm_i4g128": ([P, i32, i32, P, P, i32, P], i32),
        "lbq_quant_act_i8g128": ([P, i32, i32, P, P, P], i32),
        "lbq_gemv_i4g128_act_i8": ([P, i32, i32, P, P, i32, P], i32),
        "lbq_z80_encode": ([P, P, i32, i32, P, P], i32),
        "lbq_tern_g160_bytes": ([i32, i32], sz),
        "lbq_pack_tern_g160": ([P, P, i32, i32, P], i32),
        "lbq_unpack_tern_g160": ([P, i32, i32, P, P], i32),
        "lbq_gemv_tern_g160": ([P, i32, i32, P, P, i32, P], i32),
        "lbq_z80_chat_2bit": ([P, P, i32, P, P, i32, i32, i32, P, P, P], i32),
        "lbq_rms_rescale_bf16": ([P, P, P, i32, i32, ctypes.c_float, P], i32),
        "lbq_decode_act_elems": ([i32, i32, i32, i32, i32], sz),
        "lbq_decode_act_offset": ([i32, i32, i32, i32, i32, i32, i32], i64),
        "lbq_decode_step_q1g128": ([P, i32, i32, i32, i32, P, P, i32, ctypes.c_float, P], i32),
        "lbq_hbm_read_probe": ([P, sz, P, i32, P], i32),
        "lbq_decode_step_q1g128_noalloc": ([P, i32, i32, i32, i32, P, P, i32, ctypes.c_float,
                                            P], i32),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != LBQ_OK:
        raise LbqError(fn, status)


def _np_ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dptr(t) -> int:
    """Device pointer of a CUDA/HIP torch tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


# ------------------------------------------------------------------------------------------
# host packers (canonical numpy arrays -> device layout numpy bytes)
# ------------------------------------------------------------------------------------------

def lbq_abi_version() -> int:
    return load().lbq_abi_version()


def lbq_status_string(status: int) -> str:
    return load().lbq_status_string(status).decode()


def lbq_2bit_bytes(n: int, k: int) -> int:
    return load().lbq_2bit_bytes(n, k)


def lbq_q1g128_bytes(n: int, k: int) -> int:
    return load().lbq_q1g128_bytes(n, k)


def lbq_i4g128_bytes(n: int, k: int) -> int:
    return load().lbq_i4g128_bytes(n, k)


def lbq_pack_2bit(codes: np.ndarray) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    n, k = c.shape[0], c.shape[1] * 4
    out = np.empty(max(lbq_2bit_bytes(n, k), 1), dtype=np.uint8)
    _check("lbq_pack_2bit", load().lbq_pack_2bit(_np_ptr(c), n, k, _np_ptr(out)))
    return out


def lbq_unpack_2bit(dev: np.ndarray, n: int, k: int) -> np.ndarray:
    d = np.ascontiguousarray(dev, dtype=np.uint8)
    out = np.empty((n, k // 4), dtype=np.uint8)
    _check("lbq_unpack_2bit", load().lbq_unpack_2bit(_np_ptr(d), n, k, _np_ptr(out)))
    return out


def lbq_pack_q1g128(signs: np.ndarray, scales: np.ndarray) -> np.ndarray:
    s = np.ascontiguousarray(signs, dtype=np.uint8)
    c = np.ascontiguousarray(scales, dtype=np.uint16)
    n, k = s.shape[0], s.shape[1] * 8
    if c.shape != (n, k // 128):
        raise ValueError("scales must be [n][k/128]")
    out = np.empty(max(lbq_q1g128_bytes(n, k), 1), dtype=np.uint8)
    _check("lbq_pack_q1g128", load().lbq_pack_q1g128(_np_ptr(s), _np_ptr(c), n, k, _np_ptr(out)))
    return out


def lbq_unpack_q1g128(dev: np.ndarray, n: int, k: int):
    d = np.ascontiguousarray(dev, dtype=np.uint8)
    signs = np.empty((n, k // 8), dtype=np.uint8)
    scales = np.empty((n, k // 128), dtype=np.uint16)
    _check("lbq_unpack_q1g128",
           load().lbq_unpack_q1g128(_np_ptr(d), n, k, _np_ptr(signs), _np_ptr(scales)))
    return signs, scales


def lbq_pack_i4g128(nib: np.ndarray, scales: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(nib, dtype=np.uint8)
    c = np.ascontiguousarray(scales, dtype=np.uint16)
    n, k = q.shape[0], q.shape[1] * 2
    if c.shape != (n, k // 128):
        raise ValueError("scales must be [n][k/128]")
    out = np.empty(max(lbq_i4g128_bytes(n, k), 1), dtype=np.uint8)
    _check("lbq_pack_i4g128", load().lbq_pack_i4g128(_np_ptr(q), _np_ptr(c), n, k, _np_ptr(out)))
    return out


def lbq_unpack_i4g128(dev: np.ndarray, n: int, k: int):
    d = np.ascontiguousarray(dev, dtype=np.uint8)
    nib = np.empty((n, k // 2), dtype=np.uint8)
    scales = np.empty((n, k // 128), dtype=np.uint16)
    _check("lbq_unpack_i4g128",
           load().lbq_unpack_i4g128(_np_ptr(d), n, k, _np_ptr(nib), _np_ptr(scales)))
    return nib, scales


# ------------------------------------------------------------------------------------------
# device entry points (torch tensors in device memory)
# ------------------------------------------------------------------------------------------

def lbq_mlp_2bit_i16(layer_w, dims, x, logits, argmax=None, stream=None) -> None:
    """layer_w: list of uint8 device tensors (packed layers); x: int16 [B][dims[0]];
    logits: int16 [B][dims[-1]]; argmax: int32 [B] or None."""
    L = len(layer_w)
    ptrs = (ctypes.c_void_p * L)(*[_dptr(w) for w in layer_w])
    d = (ctypes.c_int32 * (L + 1))(*[int(v) for v in dims])
    _check("lbq_mlp_2bit_i16", load().lbq_mlp_2bit_i16(
        ctypes.cast(ptrs, ctypes.c_void_p), ctypes.cast(d, ctypes.c_void_p), L, _dptr(x),
        _dptr(logits), _dptr(argmax), x.shape[0], _stream(stream)))


def lbq_tern_g160_bytes(n: int, k: int) -> int:
    return load().lbq_tern_g160_bytes(n, k)


def lbq_pack_tern_g160(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes uint8 [n][k] in {0, 1, 2}; scales fp16 bits [n][ceil(k/160)] -> device bytes."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    n, k = codes.shape
    out = np.zeros(lbq_tern_g160_bytes(n, k), dtype=np.uint8)
    _check("lbq_pack_tern_g160", load().lbq_pack_tern_g160(_np_ptr(codes), _np_ptr(scales), n, k,
                                                           _np_ptr(out)))
    return out


def lbq_unpack_tern_g160(dev: np.ndarray, n: int, k: int):
    dev = np.ascontiguousarray(dev, dtype=np.uint8)
    codes = np.zeros((n, k), dtype=np.uint8)
    scales = np.zeros((n, (k + 159) // 160), dtype=np.uint16)
    _check("lbq_unpack_tern_g160", load().lbq_unpack_tern_g160(_np_ptr(dev), n, k, _np_ptr(codes),
                                                               _np_ptr(scales)))
    return codes, scales


def lbq_gemv_tern_g160(w, n: int, k: int, x, y, stream=None) -> None:
    B = x.shape[0] if x.dim() == 2 else 1
    _check("lbq_gemv_tern_g160", load().lbq_gemv_tern_g160(_dptr(w), n, k, _dptr(x), _dptr(y), B,
                                                           _stream(stream)))


def lbq_z80_encode(text, lengths, buckets, stream=None) -> None:
    """text: uint8 device tensor [B][stride]; lengths: int32 [B]; buckets: int16 [B][128]."""
    B, stride = text.shape
    _check("lbq_z80_encode", load().lbq_z80_encode(_dptr(text), _dptr(lengths), stride, B,
                                                   _dptr(buckets), _stream(stream)))


def lbq_z80_chat_2bit(layer_w, dims, prompts, lengths, reply, reply_len, stream=None) -> None:
    """layer_w: list of packed 2-bit layers (device); prompts: uint8 [B][stride]; lengths: int32
    [B]; reply: uint8 [B][max_reply] (output); reply_len: int32 [B] (output)."""
    L = len(layer_w)
    ptrs = (ctypes.c_void_p * L)(*[_dptr(w) for w in layer_w])
    d = (ctypes.c_int32 * (L + 1))(*[int(v) for v in dims])
    B, stride = prompts.shape
    _check("lbq_z80_chat_2bit", load().lbq_z80_chat_2bit(
        ctypes.cast(ptrs, ctypes.c_void_p), ctypes.cast(d, ctypes.c_void_p), L, _dptr(prompts),
        _dptr(lengths), stride, B, reply.shape[1], _dptr(reply) if reply.numel() else None,
        _dptr(reply_len), _stream(stream)))


def lbq_gemv_q1g128(w, n: int, k: int, x, y, stream=None) -> None:
    """w: uint8 device tensor (lbq_pack_q1g128 layout); x: bf16/int16 [B][k]; y: [B][n]."""
    B = x.shape[0] if x.dim() == 2 else 1
    _check("lbq_gemv_q1g128", load().lbq_gemv_q1g128(_dptr(w), n, k, _dptr(x), _dptr(y), B,
                                                     _stream(stream)))


def lbq_gemv_i4g128(w, n: int, k: int, x, y, stream=None) -> None:
    B = x.shape[0] if x.dim() == 2 else 1
    _check("lbq_gemv_i4g128", load().lbq_gemv_i4g128(_dptr(w), n, k, _dptr(x), _dptr(y), B,
                                                     _stream(stream)))


def lbq_gemm_q1g128(w, n: int, k: int, x, y, stream=None) -> None:
    """Many-row product on the matrix cores. w: lbq_pack_q1g128 layout; x: bf16/int16 [m][k]
    (16-byte aligned); y: [m][n]."""
    m = x.shape[0] if x.dim() == 2 else 1
    _check("lbq_gemm_q1g128", load().lbq_gemm_q1g128(_dptr(w), n, k, _dptr(x), _dptr(y), m,
                                                     _stream(stream)))


def lbq_gemm_i4g128(w, n: int, k: int, x, y, stream=None) -> None:
    m = x.shape[0] if x.dim() == 2 else 1
    _check("lbq_gemm_i4g128", load().lbq_gemm_i4g128(_dptr(w), n, k, _dptr(x), _dptr(y), m,
                                                     _stream(stream)))


def lbq_quant_act_i8g128(x, q, scale, stream=None) -> None:
    """x: bf16/int16 [B][k] -> q: int8 [B][k], scale: float32 [B][k/128] (all device tensors)."""
    B, k = (x.shape[0], x.shape[1]) if x.dim() == 2 else (1, x.shape[0])
    _check("lbq_quant_act_i8g128", load().lbq_quant_act_i8g128(
        _dptr(x), k, B, _dptr(q), _dptr(scale), _stream(stream)))


def lbq_gemv_i4g128_act_i8(w, n: int, k: int, x, y, stream=None) -> None:
    """INT4 weights x int8-quantized activations (quantized in the kernel). x: bf16 [B][k]."""
    B = x.shape[0] if x.dim() == 2 else 1
    _check("lbq_gemv_i4g128_act_i8", load().lbq_gemv_i4g128_act_i8(
        _dptr(w), n, k, _dptr(x), _dptr(y), B, _stream(stream)))


def lbq_rms_rescale_bf16(y, x, y2=None, eps: float = 1e-6, stream=None) -> None:
    B, n = (y.shape[0], y.shape[1]) if y.dim() == 2 else (1, y.shape[0])
    _check("lbq_rms_rescale_bf16", load().lbq_rms_rescale_bf16(
        _dptr(y), _dptr(y2), _dptr(x), n, B, float(eps), _stream(stream)))


def lbq_decode_act_elems(n_layers, hidden, kv, ffn, batch) -> int:
    return load().lbq_decode_act_elems(n_layers, hidden, kv, ffn, batch)


def lbq_decode_act_offset(layer, slot, n_layers, hidden, kv, ffn, batch) -> int:
    return load().lbq_decode_act_offset(layer, slot, n_layers, hidden, kv, ffn, batch)


def make_layers(layers) -> ctypes.Array:
    """layers: list of dicts {name: uint8 device tensor} -> lbq_q1_layer array. The array holds
    references to the tensors, so their memory stays allocated while the array is in use."""
    arr = (Q1Layer * len(layers))()
    for i, L in enumerate(layers):
        for name in ("q", "k", "v", "o", "gate", "up", "down"):
            setattr(arr[i], name, _dptr(L[name]))
    arr._tensors = [dict(L) for L in layers]
    return arr


def lbq_decode_step_q1g128(layer_array, n_layers, hidden, kv, ffn, x0, act, eps=1e-6,
                           stream=None) -> None:
    B = x0.shape[0]
    _check("lbq_decode_step_q1g128", load().lbq_decode_step_q1g128(
        ctypes.cast(layer_array, ctypes.c_void_p), n_layers, hidden, kv, ffn, _dptr(x0),
        _dptr(act), B, float(eps), _stream(stream)))


def lbq_decode_step_q1g128_noalloc(layer_array, n_layers, hidden, kv, ffn, x0, act, eps=1e-6,
                                   stream=None) -> None:
    B = x0.shape[0]
    _check("lbq_decode_step_q1g128_noalloc", load().lbq_decode_step_q1g128_noalloc(
        ctypes.cast(layer_array, ctypes.c_void_p), n_layers, hidden, kv, ffn, _dptr(x0),
        _dptr(act), B, float(eps), _stream(stream)))


def lbq_hbm_read_probe(src, sink, workgroups: int, stream=None) -> None:
    """Streams every byte of the device tensor `src` once (bandwidth reference)."""
    nbytes = src.numel() * src.element_size()
    _check("lbq_hbm_read_probe", load().lbq_hbm_read_probe(
        _dptr(src), nbytes, _dptr(sink), int(workgroups), _stream(stream)))


def act_view(act, slot: str, layer: int, n_layers, hidden, kv, ffn, batch):
    """[batch][dim] view of one slot of the decode-step activation record."""
    idx = ACT_SLOTS.index(slot) if slot != "final" else len(ACT_SLOTS)
    off = lbq_decode_act_offset(layer, idx, n_layers, hidden, kv, ffn, batch)
    dim = {"x": hidden, "q": hidden, "k": kv, "v": kv, "gate": ffn, "up": ffn, "xo": hidden,
           "o": hidden, "xd": ffn, "down": hidden, "final": hidden}[slot]
    return act[off:off + batch * dim].view(batch, dim)
