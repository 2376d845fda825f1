"""Oracle runs over whole synthetic workloads (test infrastructure only).

Each function regenerates its inputs from ``workloads`` and calls
``oracle.decode``; nothing here takes values from the GPU path except the
explicit teacher-forcing arguments (``x_in``), which tests use to check one
layer at a time.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple

import numpy as np

import workloads as wl
from . import decode as od
from . import prefill as op


def pools_f64(w: "wl.Workload", layer: int) -> Tuple[np.ndarray, np.ndarray]:
    k, v = w.kv(layer)
    return k.astype(np.float64), v.astype(np.float64)


def layer_batch(w: "wl.Workload", layer: int, x_in: np.ndarray,
                pools: Optional[Tuple[np.ndarray, np.ndarray]] = None,
                weights=None, exact: bool = False, mirror: bool = False,
                rows: Optional[np.ndarray] = None):
    """Run one layer for the sequences `rows` of the batch (default: all);
    x_in [len(rows), H]. Returns (x_out [len(rows), H], k_pool, v_pool) with
    the pools (float64) holding the written slots.

    The steps of decode.decode_layer, each applied to the whole batch at once
    where it is per-row (RMSNorm, projections, RoPE, SiLU-mul, residuals) and
    per sequence for the page writes and the attention; every sequence owns
    its pages and slots, so writing all new K/V before any attention equals
    running the sequences one after another."""
    sh = w.shape
    lw = weights if weights is not None else w.layer(layer)
    kp, vp = pools if pools is not None else pools_f64(w, layer)
    rows = np.arange(w.batch) if rows is None else np.asarray(rows)
    x = np.asarray(x_in, dtype=np.float64).reshape(len(rows), sh.hidden)
    pos = w.positions[rows]
    q, k, v = od.qkv_stage(x, lw, pos, sh, exact, mirror)
    for i, b in enumerate(rows):
        od.kv_write(kp, vp, w.page_tables[b], int(pos[i]), k[i], v[i])
    o = np.stack([od.attention_decode(q[i], kp, vp, w.page_tables[b], int(w.ctx_lens[b]), exact)
                  for i, b in enumerate(rows)])
    x1 = od.oproj_stage(x, o.reshape(len(rows), -1), lw, exact)
    h = od.gate_up_stage(x1, lw, sh, exact, mirror)
    return od.down_stage(x1, h, lw, exact), kp, vp


def attention_batch(w: "wl.Workload", q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                    exact: bool = False) -> np.ndarray:
    """Attention only: o [B, Hq, D] for every sequence."""
    kp = np.asarray(k_pool, dtype=np.float64)
    vp = np.asarray(v_pool, dtype=np.float64)
    return np.stack([od.attention_decode(q[b], kp, vp, w.page_tables[b], int(w.ctx_lens[b]), exact)
                     for b in range(w.batch)])


def lm_head_rows(w: "wl.Workload", xf: np.ndarray, rows: Optional[np.ndarray] = None,
                 exact: bool = False) -> np.ndarray:
    """r(W_lm xf) for the given vocab rows (all rows by default); xf [B, H]
    is the final-normed input. W_lm is regenerated chunk by chunk."""
    sh = w.shape
    rows = np.arange(sh.vocab) if rows is None else np.asarray(rows)
    out = np.empty((xf.shape[0], len(rows)), dtype=np.float64)
    chunks = rows // wl.ROW_CHUNK
    for c in np.unique(chunks):
        blk = wl.lm_head_chunk(w.workload_id, sh, int(c)).astype(np.float64)
        sel = np.nonzero(chunks == c)[0]
        out[:, sel] = (blk[rows[sel] - c * wl.ROW_CHUNK] @ xf.T).T
    return od.r16(out, exact)


def step(w: "wl.Workload", layers: Optional[int] = None, logits_rows: Optional[np.ndarray] = None,
         keep_residuals: bool = False, progress=None, exact: bool = False,
         mirror: bool = False) -> Dict[str, np.ndarray]:
    """Full decode step: x = E[token]; decoder layers; final RMSNorm; lm_head.

    Returns {"logits": [B, n_rows], "x_final": [B, H], "residuals": [L+1, B, H]?}.
    `layers` < n_layers truncates the stack (for bounded CPU-baseline samples).
    """
    sh = w.shape
    nl = sh.n_layers if layers is None else layers
    tokens = w.tokens()
    x = wl.embedding_rows(w.workload_id, sh, tokens).astype(np.float64)
    res = [x.copy()] if keep_residuals else None
    for l in range(nl):
        x, _, _ = layer_batch(w, l, x, exact=exact, mirror=mirror)
        if keep_residuals:
            res.append(x.copy())
        if progress:
            progress(l)
    xf = np.stack([od.rmsnorm(x[b], w.final_norm(), sh.eps, exact) for b in range(w.batch)])
    out = {"x_final": x, "xf": xf, "logits": lm_head_rows(w, xf, logits_rows, exact)}
    if keep_residuals:
        out["residuals"] = np.stack(res)
    return out


def prefill_run(w: "wl.Workload", tokens: np.ndarray, start: int = 0, layers: Optional[int] = None,
                exact: bool = False, mirror: bool = False, keep_pools: bool = False):
    """Prefill of the prompt `tokens` for sequence 0 of the workload (its page
    table row), positions start .. start + n - 1, over the workload's
    generated pages. Returns {"logits": [V] of the last token, "x": [n, H]
    final residual rows, "pools": [(k_pool, v_pool)] per layer (keep_pools)}."""
    sh = w.shape
    nl = sh.n_layers if layers is None else layers
    x = wl.embedding_rows(w.workload_id, sh, np.asarray(tokens)).astype(np.float64)
    pt = w.page_tables[0]
    pools = []
    for l in range(nl):
        kp, vp = pools_f64(w, l)
        x = op.prefill_layer(x, w.layer(l), kp, vp, pt, start, sh, exact, mirror)
        if keep_pools:
            pools.append((kp, vp))
    xf = od.rmsnorm(x[-1:], w.final_norm(), sh.eps, exact)
    out = {"logits": lm_head_rows(w, xf, exact=exact)[0], "x": x}
    if keep_pools:
        out["pools"] = pools
    return out

