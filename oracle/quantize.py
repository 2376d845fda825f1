"""Symmetric group-wise INT4 quantisation of fp16 weights (test
infrastructure only; see the package header).

Source: "How to build your own LLM runtime from scratch", "Architectural
decisions and optimizations": the weights are quantised symmetrically and
group-wise to INT4 with groups of 128.

Readings where the pages are silent:
  * groups run along the input dimension (the same groups the dequantisation
    w = q * s uses), the last group of a row partial when k is not a multiple
    of 128;
  * the scale of a (row, group) is the fp16 value nearest to max|w| / 7, so the
    largest magnitude maps to code +-7 (symmetric: code -8 is not produced);
  * the code is the integer in [-8, 7] nearest to w / s, halfway cases to the
    even integer; a group whose scale is 0 (all zeros, or a maximum too small
    for fp16) gets codes 0;
  * weights must be finite.
"""
from __future__ import annotations

import numpy as np

GROUP = 128


def quantize_w4g128(w: np.ndarray):
    """w: fp16 [n, k] -> (q int8 [n, k], s fp16 [n, ceil(k / 128)])."""
    w = np.asarray(w)
    assert w.dtype == np.float16 and w.ndim == 2
    wf = w.astype(np.float64)
    assert np.isfinite(wf).all()
    n, k = wf.shape
    groups = (k + GROUP - 1) // GROUP
    q = np.zeros((n, k), dtype=np.int8)
    s = np.zeros((n, groups), dtype=np.float16)
    for g in range(groups):
        lo, hi = GROUP * g, min(k, GROUP * g + GROUP)
        block = wf[:, lo:hi]
        scale = (np.abs(block).max(axis=1) / 7.0).astype(np.float16)   # nearest fp16
        s[:, g] = scale
        sf = scale.astype(np.float64)[:, None]
        ratio = np.zeros_like(block)
        np.divide(block, sf, out=ratio, where=sf > 0)
        q[:, lo:hi] = np.clip(np.rint(ratio), -8, 7).astype(np.int8)     # rint: halves to even
    return q, s
