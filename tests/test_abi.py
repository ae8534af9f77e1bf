"""CPU tests of the library boundary: the shared library loads without a GPU and exports every
function include/lbq.h declares; host packers are exact inverses of their unpackers and have
the documented sizes; argument validation rejects bad calls before any device work."""
import ctypes
import os
import re

import numpy as np
import pytest

import packed_weight_gemv_amd as lbq
from packed_weight_gemv_amd import synth


def _declared_functions():
    src = open(lbq.HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(lbq_[a-z0-9_]+)\s*\(", src)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    return lbq.load()


def test_library_exports_every_declared_function(lib):
    names = _declared_functions()
    assert len(names) == 30
    for name in names:
        assert hasattr(lib, name), name
        assert name in dir(lbq) or name in ("lbq_status_string",), f"binding lacks {name}"


def test_abi_version_and_status_strings(lib):
    assert lbq.lbq_abi_version() == 2
    for code in lbq.STATUS:
        assert lbq.lbq_status_string(code)
    assert lbq.lbq_status_string(12345) == "unknown status"


def test_q1_bytes_closed_form():
    # 1.125 bits per weight, no padding when n % 64 == 0 and k % 1024 == 0
    for n, k in ((5120, 5120), (1024, 5120), (17408, 5120), (5120, 17408)):
        assert lbq.lbq_q1g128_bytes(n, k) == n * k * 9 // 64
    assert lbq.lbq_q1g128_bytes(5120, 5120) == 3686400
    assert lbq.lbq_q1g128_bytes(17408, 5120) == 12533760
    # ragged rows and k pad up, never down
    assert lbq.lbq_q1g128_bytes(65, 128) >= 65 * 128 * 9 // 64
    for bad in ((0, 128), (64, 0), (64, 100), (64, 129)):
        assert lbq.lbq_q1g128_bytes(*bad) == 0


def test_i4_and_2bit_bytes_closed_forms():
    for n, k in ((4096, 4096), (1024, 4096), (12288, 4096), (4096, 12288)):
        assert lbq.lbq_i4g128_bytes(n, k) == n * k * 33 // 64
    assert lbq.lbq_i4g128_bytes(4096, 4096) == 8650752
    assert lbq.lbq_i4g128_bytes(12288, 4096) == 25952256
    assert lbq.lbq_2bit_bytes(192, 256) == 192 * 64
    total = sum(lbq.lbq_2bit_bytes(n, k) for k, n in zip(synth.MLP_DIMS, synth.MLP_DIMS[1:]))
    assert total == 19712


@pytest.mark.parametrize("n,k", [(64, 1024), (70, 1152), (1, 128), (130, 2176)])
def test_q1_pack_roundtrip(n, k):
    m = synth.q1_matrix(n, k, workload=60)
    dev = lbq.lbq_pack_q1g128(m.signs, m.scales)
    assert dev.size == lbq.lbq_q1g128_bytes(n, k)
    s2, c2 = lbq.lbq_unpack_q1g128(dev, n, k)
    assert np.array_equal(s2, m.signs) and np.array_equal(c2, m.scales)


@pytest.mark.parametrize("n,k", [(64, 1024), (70, 1152), (1, 128), (130, 2176)])
def test_i4_pack_roundtrip(n, k):
    m = synth.i4_matrix(n, k, workload=61)
    dev = lbq.lbq_pack_i4g128(m.nib, m.scales)
    assert dev.size == lbq.lbq_i4g128_bytes(n, k)
    q2, c2 = lbq.lbq_unpack_i4g128(dev, n, k)
    assert np.array_equal(q2, m.nib) and np.array_equal(c2, m.scales)


def test_2bit_pack_roundtrip():
    codes = synth.mlp2bit_layers()[0]
    dev = lbq.lbq_pack_2bit(codes)
    assert np.array_equal(lbq.lbq_unpack_2bit(dev, codes.shape[0], codes.shape[1] * 4), codes)


def test_q1_device_layout_places_scales_next_to_their_groups():
    # one tile, one super-group: first 1 KiB = 64 rows x 8 fp16 scales, then 1 KiB per group
    m = synth.q1_matrix(64, 1024, workload=62)
    dev = lbq.lbq_pack_q1g128(m.signs, m.scales)
    sc = dev[:1024].view(np.uint16).reshape(64, 8)
    assert np.array_equal(sc, m.scales)
    rec = dev[1024:2048].view(np.uint32).reshape(64, 4)
    canon = m.signs[:, :16].copy().view(np.uint32).reshape(64, 4)
    rot = ((canon << np.uint32(2)) | (canon >> np.uint32(30))).astype(np.uint32)
    assert np.array_equal(rec, rot)


def test_packers_reject_bad_shapes(lib):
    buf = np.zeros(1 << 16, dtype=np.uint8)
    sc = np.zeros(1 << 12, dtype=np.uint16)
    p = buf.ctypes.data
    assert lib.lbq_pack_q1g128(p, sc.ctypes.data, 64, 100, p) == -2
    assert lib.lbq_pack_q1g128(None, sc.ctypes.data, 64, 128, p) == -1
    assert lib.lbq_pack_i4g128(p, sc.ctypes.data, 0, 128, p) == -2
    assert lib.lbq_pack_2bit(p, 4, 6, p) == -2


def test_device_entry_points_validate_before_touching_the_device(lib):
    # NULL pointers, bad shapes, misalignment and aliasing are reported without a launch
    fake = 1 << 40           # never dereferenced: validation fails first
    assert lib.lbq_gemv_q1g128(None, 64, 128, fake, fake + 4096, 1, None) == -1
    assert lib.lbq_gemv_q1g128(fake, 64, 100, fake + 4096, fake + 8192, 1, None) == -2
    assert lib.lbq_gemv_q1g128(fake, 64, 128, fake + 4096, fake + 8192, 17, None) == -2
    assert lib.lbq_gemv_q1g128(fake + 8, 64, 128, fake + 4096, fake + 8192, 1, None) == -3
    assert lib.lbq_gemv_q1g128(fake, 64, 128, fake + (1 << 20), fake + (1 << 20) + 64, 1, None) == -5
    assert lib.lbq_gemv_i4g128(fake, 64, 128, fake + 4098, fake + 8192, 1, None) == -3
    assert lib.lbq_rms_rescale_bf16(fake, None, fake + 2, 64, 1, ctypes.c_float(1e-6), None) == -5
    assert lib.lbq_rms_rescale_bf16(fake, None, fake + 4096, 64, 1, ctypes.c_float(-1.0), None) == -2
    dims = (ctypes.c_int32 * 2)(6, 4)
    ws = (ctypes.c_void_p * 1)(fake)
    assert lib.lbq_mlp_2bit_i16(ws, dims, 1, fake + 4096, fake + 8192, None, 1, None) == -2
    dims2 = (ctypes.c_int32 * 2)(8, 4)
    assert lib.lbq_mlp_2bit_i16(ws, dims2, 1, fake + 4096, fake + 4096, None, 1, None) == -5
    assert lib.lbq_mlp_2bit_i16(ws, dims2, 9, fake + 4096, fake + 8192, None, 1, None) == -2


def test_decode_activation_record_geometry():
    L, h, kv, f, B = 3, 256, 128, 384, 2
    per_layer = B * (h + h + kv + kv + f + f + h + h + f + h)
    assert lbq.lbq_decode_act_elems(L, h, kv, f, B) == per_layer * L + B * h
    assert lbq.lbq_decode_act_offset(0, 0, L, h, kv, f, B) == 0
    assert lbq.lbq_decode_act_offset(1, 0, L, h, kv, f, B) == per_layer
    assert lbq.lbq_decode_act_offset(0, 2, L, h, kv, f, B) == 2 * B * h
    assert lbq.lbq_decode_act_offset(L, 10, L, h, kv, f, B) == per_layer * L
    assert lbq.lbq_decode_act_offset(L, 3, L, h, kv, f, B) == -1
    assert lbq.lbq_decode_act_elems(L, 100, kv, f, B) == 0


@pytest.mark.parametrize("n,k", [(64, 160), (70, 1000), (1, 37), (130, 17408), (3, 1281)])
def test_tern_pack_roundtrip(n, k):
    m = synth.tern_matrix(n, k, matrix=n + k)
    dev = lbq.lbq_pack_tern_g160(m.codes, m.scales)
    assert dev.size == lbq.lbq_tern_g160_bytes(n, k)
    c2, s2 = lbq.lbq_unpack_tern_g160(dev, n, k)
    assert np.array_equal(c2, m.codes) and np.array_equal(s2, m.scales)


def test_tern_sizes_and_digit_order():
    # 1.7 bits per weight on aligned shapes (34 bytes per 160 weights)
    for n, k in ((5120, 5120), (1024, 5120), (17408, 5120)):
        assert lbq.lbq_tern_g160_bytes(n, k) == n * k // 160 * 34
    n, k = 64, 160
    codes = np.ones((n, k), dtype=np.uint8)
    codes[0, :5] = [2, 0, 1, 1, 2]            # byte 0 of row 0: 2 + 0*3 + 1*9 + 1*27 + 2*81
    codes[1, 5:10] = [0, 0, 0, 0, 0]          # byte 1 of row 1: 0
    scales = np.arange(n, dtype=np.uint16)[:, None]
    dev = lbq.lbq_pack_tern_g160(codes, scales)
    assert np.array_equal(dev[:1024].view(np.uint16).reshape(64, 8)[:, 0], scales[:, 0])
    rec = dev[1024:2048].reshape(64, 16)      # bytes 0..15 of every row's group record
    assert rec[0, 0] == 2 + 9 + 27 + 162 and rec[1, 1] == 0 and rec[2, 0] == 121
    # a code above 2 is rejected
    bad = codes.copy()
    bad[5, 7] = 3
    with pytest.raises(lbq.LbqError) as e:
        lbq.lbq_pack_tern_g160(bad, scales)
    assert e.value.status == -8
