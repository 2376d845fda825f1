"""Reads the library's packed weight formats back into plain arrays (test
infrastructure only; see package header).

Written from the format description alone (the "w4g128" and packed-fp16
layouts documented with the packing entry points of the C interface), with
explicit per-field loops over tiles and lanes, so a packing mistake shows up
as a mismatch against the generator's (q, s).
"""
from __future__ import annotations

import numpy as np

ROLE_PLAIN, ROLE_QKV, ROLE_GATE_UP = 0, 1, 2


def logical_rows(n: int, role: int, head_dim: int = 0) -> np.ndarray:
    """Logical row held by each physical row (padding rows -> -1)."""
    t = (n + 15) // 16
    phys = np.full(16 * t, -1, dtype=np.int64)
    if role == ROLE_PLAIN:
        phys[:n] = np.arange(n)
    elif role == ROLE_QKV:
        d = head_dim
        for head in range(n // d):
            for p in range(d // 16):
                base = head * d + 16 * p
                for i in range(8):
                    phys[base + i] = head * d + 8 * p + i
                    phys[base + 8 + i] = head * d + d // 2 + 8 * p + i
    elif role == ROLE_GATE_UP:
        f = n // 2
        for tt in range(f // 8):
            for i in range(8):
                phys[16 * tt + i] = 8 * tt + i
                phys[16 * tt + 8 + i] = f + 8 * tt + i
    else:
        raise ValueError(role)
    return phys


def column_of_nibble(bit: int) -> int:
    """Offset e (0..7) inside a 32-bit word of the nibble starting at `bit`."""
    if bit < 16:
        return 2 * (bit // 4)
    return 2 * ((bit - 16) // 4) + 1


def unpack_w4g128(buf: bytes, n: int, k: int, role: int, head_dim: int = 0):
    """Return (q int8 [n, k], s fp16 [n, ceil(k/128)]) from a packed buffer,
    plus the padding contents (q of padding columns/rows, s of padding rows)
    so tests can check they are exactly 0."""
    t_tiles = (n + 15) // 16
    g_groups = (k + 127) // 128
    raw = np.frombuffer(buf, dtype=np.uint8)
    words = raw[: t_tiles * g_groups * 1024].view("<u4").reshape(t_tiles, g_groups, 64, 4)
    scales = raw[t_tiles * g_groups * 1024: t_tiles * g_groups * 1024 + t_tiles * g_groups * 32]
    scales = scales.view("<u2").reshape(t_tiles, g_groups, 16)
    rows = logical_rows(n, role, head_dim)
    kp = 128 * g_groups
    qp = np.zeros((16 * t_tiles, kp), dtype=np.int16)     # physical rows, padded columns
    for lane in range(64):
        prow_in_tile = lane & 15
        c0 = 32 * (lane >> 4)
        for j in range(4):
            w = words[:, :, lane, j].astype(np.uint64)    # [T, G]
            for bit in range(0, 32, 4):
                u = ((w >> np.uint64(bit)) & np.uint64(15)).astype(np.int16)
                col = c0 + 8 * j + column_of_nibble(bit)
                for g in range(g_groups):
                    qp[prow_in_tile::16, 128 * g + col] = u[:, g] - 8
    sp = scales.transpose(0, 2, 1).reshape(16 * t_tiles, g_groups)   # [physical row, group]
    q = np.zeros((n, k), dtype=np.int8)
    s = np.zeros((n, g_groups), dtype=np.uint16)
    live = rows >= 0
    q[rows[live]] = qp[live, :k]
    s[rows[live]] = sp[live]
    pad_q = np.concatenate([qp[live, k:].ravel(), qp[~live].ravel()])
    pad_s = sp[~live].ravel()
    return q, s.view(np.float16), pad_q, pad_s


def unpack_f16(buf: bytes, n: int, k: int):
    """Return (w fp16 [n, k], padding values) from a packed-fp16 buffer."""
    t_tiles = (n + 15) // 16
    c_blocks = (k + 31) // 32
    h = np.frombuffer(buf, dtype="<u2")[: t_tiles * c_blocks * 512].reshape(t_tiles, c_blocks, 64, 8)
    wp = np.zeros((16 * t_tiles, 32 * c_blocks), dtype=np.uint16)
    for lane in range(64):
        for c in range(c_blocks):
            col = 32 * c + 8 * (lane >> 4)
            wp[(lane & 15)::16, col:col + 8] = h[:, c, lane, :]
    pad = np.concatenate([wp[:n, k:].ravel(), wp[n:].ravel()])
    return wp[:n, :k].view(np.float16), pad.view(np.float16)
