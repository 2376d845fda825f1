"""W4A8 variant of the projections (test infrastructure only; see package header).

The pages report that an INT8-activation path (__dp4a) lost to unpacking the
INT4 weights for 16-bit math on Hopper ("How to build your own LLM runtime
from scratch", Architectural decisions and optimizations: prmt.b32 versus
__dp4a for the gate/up/down GEMVs). The variant measured here against the
W4A16 projections quantises each activation row to INT8 and multiplies
integers. The pages do not say how the activations were quantised; the
reading is the plainest symmetric one:

  s_x = max_k |x_k| / 127 (float32), x_q = round(x / s_x) to the nearest
  integer (halves to even), clamped to [-127, 127]; a row of zeros has
  s_x = 0 and x_q = 0.
  y[n] = s_x * sum_g s[n, g] * sum_{k in g} q[n, k] * x_q[k]   (integer inner sums)

The code decision (which integer x_q is) is taken in float32, as the kernel
takes it; everything after it is exact integers or float64 here. Outputs are
rounded once to fp16.
"""
from __future__ import annotations

import numpy as np

from . import decode as od

GROUP = od.GROUP


def quantize_rows_int8(x: np.ndarray):
    """(x_q int32 [..., K] in [-127, 127], s_x float32 [...]) per row of fp16 x."""
    xf = np.asarray(x, dtype=np.float16).astype(np.float32)
    amax = np.abs(xf).max(axis=-1)
    s = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    with np.errstate(invalid="ignore"):
        xq = np.rint((xf / safe[..., None]).astype(np.float32))
    xq = np.clip(np.where(s[..., None] > 0, xq, 0), -127, 127).astype(np.int32)
    return xq, s


def gemv_w4a8(q: np.ndarray, s: np.ndarray, x: np.ndarray) -> np.ndarray:
    """r(y) for y = W4A8 product of packed-format-free (q, s) with fp16 rows x [..., K]."""
    x = np.asarray(x)
    lead = x.shape[:-1]
    xb = x.reshape(-1, x.shape[-1])
    xq, sx = quantize_rows_int8(xb)
    n, k = q.shape
    ng = (k + GROUP - 1) // GROUP
    y = np.zeros((xb.shape[0], n), dtype=np.float64)
    qf = q.astype(np.float64)
    xf = xq.astype(np.float64)
    for g in range(ng):
        c0, c1 = g * GROUP, min(k, (g + 1) * GROUP)
        # integer products summed in float64: every partial sum is an integer
        # below 2^17, so the sum is exact
        part = xf[:, c0:c1] @ qf[:, c0:c1].T
        y += part * np.asarray(s[:, g], dtype=np.float64)[None, :]
    y *= sx.astype(np.float64)[:, None]
    return od.r16(y).reshape(lead + (n,))
