"""Packer: pack (C library) -> independent reader (oracle.packing) round trips
bit-exactly; hand-derived bytes pin the documented layout (CPU only)."""
import numpy as np
import pytest

import w4a16_paged_kv_amd as w4
import workloads as wl
from oracle import packing as op


def _rand(n, k, seed=0):
    g = np.random.default_rng(seed)
    q = g.integers(-8, 8, (n, k)).astype(np.int8)
    s = wl.group_scales(g, n, k)
    return q, s


@pytest.mark.parametrize("n,k,role,hd", [
    (16, 128, w4.ROLE_PLAIN, 0), (37, 448, w4.ROLE_PLAIN, 0), (448, 1536, w4.ROLE_PLAIN, 0),
    (576, 448, w4.ROLE_QKV, 64), (4608 // 8, 256, w4.ROLE_QKV, 64), (9 * 128, 384, w4.ROLE_QKV, 128),
    (3072, 448, w4.ROLE_GATE_UP, 0), (2 * 72, 200, w4.ROLE_GATE_UP, 0), (5, 8, w4.ROLE_PLAIN, 0)])
def test_roundtrip_bit_exact(n, k, role, hd):
    q, s = _rand(n, k, n * 1000 + k)
    buf = w4.pack_weights_w4g128(q, s, role, hd)
    assert buf.size == w4.w4_packed_bytes(n, k) == ((n + 15) // 16) * ((k + 127) // 128) * 1056
    q2, s2, pad_q, pad_s = op.unpack_w4g128(buf.tobytes(), n, k, role, hd)
    assert np.array_equal(q2, q)
    assert np.array_equal(s2.view(np.uint16), s.view(np.uint16))
    assert np.all(pad_q == 0) and np.all(pad_s == 0)


def test_pack_is_deterministic():
    q, s = _rand(64, 300, 1)
    assert np.array_equal(w4.pack_weights_w4g128(q, s), w4.pack_weights_w4g128(q, s))


def test_hand_derived_bytes():
    """N = 1, K = 128, q[0, k] = (k % 16) - 8, s = 1.0 (0x3c00).
    Lane 0 (row 0, columns 0..31), word 0 holds columns 0..7 = codes u = 0..7;
    even offsets go to bits 0,4,8,12 and odd ones to bits 16,20,24,28, so
    word 0 = u0 | u2<<4 | u4<<8 | u6<<12 | u1<<16 | u3<<20 | u5<<24 | u7<<28
           = 0x7531_6420 (little-endian bytes 20 64 31 75).
    Word 1 holds columns 8..15 (u = 8..15): 0xFDB9_ECA8.
    Lane 16 is row 0, columns 32..63 (same codes). Rows 1..15 are padding
    (u = 8 everywhere: bytes 0x88). The scale section starts at byte 1024."""
    q = (np.arange(128) % 16 - 8).astype(np.int8)[None, :]
    s = np.array([[1.0]], dtype=np.float16)
    b = w4.pack_weights_w4g128(q, s)
    assert list(b[0:4]) == [0x20, 0x64, 0x31, 0x75]
    assert list(b[4:8]) == [0xA8, 0xEC, 0xB9, 0xFD]
    assert list(b[16 * 16: 16 * 16 + 8]) == [0x20, 0x64, 0x31, 0x75, 0xA8, 0xEC, 0xB9, 0xFD]
    assert np.all(b[16:32] == 0x88)                         # lane 1 = padding row 1
    assert list(b[1024:1026]) == [0x00, 0x3C] and np.all(b[1026:1056] == 0)


def test_hand_derived_role_orders():
    # QKV role, head_dim 32: physical rows 0..7 = dims 0..7, rows 8..15 = dims 16..23
    rows = op.logical_rows(64, w4.ROLE_QKV, 32)
    assert list(rows[:16]) == list(range(8)) + list(range(16, 24))
    assert list(rows[16:32]) == list(range(8, 16)) + list(range(24, 32))
    assert list(rows[32:48]) == [32 + r for r in list(range(8)) + list(range(16, 24))]
    # GATE_UP role, F = 24: tile 1 = gate 8..15 then up 32..39
    rows = op.logical_rows(48, w4.ROLE_GATE_UP)
    assert list(rows[16:32]) == list(range(8, 16)) + list(range(32, 40))


def test_out_of_range_code_is_rejected():
    q, s = _rand(16, 128)
    q[3, 7] = 8
    with pytest.raises(w4.W4Error) as e:
        w4.pack_weights_w4g128(q, s)
    assert e.value.code == w4.W4_ERANGE
    q[3, 7] = -9
    with pytest.raises(w4.W4Error):
        w4.pack_weights_w4g128(q, s)


def test_bad_roles_and_shapes():
    q, s = _rand(24, 128)
    with pytest.raises(w4.W4Error) as e:
        w4.pack_weights_w4g128(q, s, w4.ROLE_GATE_UP)        # n = 2F needs F % 8 == 0
    assert e.value.code == w4.W4_EINVAL
    with pytest.raises(w4.W4Error):
        w4.pack_weights_w4g128(q, s, w4.ROLE_QKV, 20)        # head_dim % 16
    with pytest.raises(w4.W4Error):
        w4.pack_weights_w4g128(q, s, 7)
    assert w4.w4_packed_bytes(0, 5) == 0


@pytest.mark.parametrize("n,k", [(16, 32), (37, 448), (152, 3584 // 4), (3, 8)])
def test_f16_roundtrip(n, k):
    wgt = np.random.default_rng(n).standard_normal((n, k)).astype(np.float16)
    buf = w4.pack_weights_f16(wgt)
    assert buf.size == w4.w4_packed_f16_bytes(n, k)
    w2, pad = op.unpack_f16(buf.tobytes(), n, k)
    assert np.array_equal(w2.view(np.uint16), wgt.view(np.uint16))
    assert np.all(pad == 0)


def test_f16_hand_derived_bytes():
    """Lane 17 = row 1, columns 8..15 -> bytes [272, 288) hold w[1, 8:16]."""
    wgt = np.arange(2 * 32, dtype=np.float16).reshape(2, 32)
    b = w4.pack_weights_f16(wgt).view(np.float16)
    assert np.array_equal(b[17 * 8: 18 * 8], wgt[1, 8:16])
    assert np.array_equal(b[0:8], wgt[0, 0:8])
