"""Prefill of a prompt in float64 (test infrastructure only; see package header).

Before decoding, the runtime runs the whole prompt through the model once:
every prompt token's K and V are written into the sequence's pages, and the
last token's logits give the first generated token ("How to build your own
LLM runtime from scratch", Key performance metrics: time to first token for a
512-token prompt). The pages give no algorithm beyond that; the reading is
the plainest one: token i of the prompt sits at position start + i, and every
layer applies, to every prompt row at once, the same steps as one decode
step (oracle.decode) -- RMSNorm, the qkv projection, RoPE at the row's own
position, the K/V write into page page_table[p // 16], slot p % 16, causal
attention over positions [0, p] (the row's own K/V included, earlier
prompt rows and any prior context already in the pages), the o projection
with its residual, RMSNorm, SiLU-gated MLP, residual. Each row is thus
exactly the decode step of its token, and rows interact only through the
pages; the pins check that prefill equals that many decode steps run one
after another.
"""
from __future__ import annotations

import numpy as np

from . import decode as od


def prefill_layer(x: np.ndarray, w, k_pool: np.ndarray, v_pool: np.ndarray,
                  page_table_row: np.ndarray, start: int, shape, exact: bool = False,
                  mirror: bool = False) -> np.ndarray:
    """One layer over the prompt rows x [n, H] at positions start .. start+n-1.
    Updates the float64 pools in place with every row's K and V and returns
    the new residual rows [n, H]."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    pos = start + np.arange(n)
    q, k, v = od.qkv_stage(x, w, pos, shape, exact, mirror)
    for i in range(n):
        od.kv_write(k_pool, v_pool, page_table_row, int(pos[i]), k[i], v[i])
    # causal: row i reads positions [0, start + i], i.e. ctx = start + i + 1
    o = np.stack([od.attention_decode(q[i], k_pool, v_pool, page_table_row, int(pos[i]) + 1, exact)
                  for i in range(n)])
    x1 = od.oproj_stage(x, o.reshape(n, -1), w, exact)
    h = od.gate_up_stage(x1, w, shape, exact, mirror)
    return od.down_stage(x1, h, w, exact)


def prefill(x0: np.ndarray, layer_weights, pools, page_table_row: np.ndarray, start: int, shape,
            final_norm: np.ndarray, lm_head_rows, exact: bool = False, mirror: bool = False):
    """The whole prompt: x0 [n, H] (embedding rows of the prompt tokens)
    through the layers (layer_weights[l], pools[l] = (k_pool, v_pool), both
    updated in place), then the final RMSNorm and the fp16 lm_head of the
    last row. lm_head_rows(xf [1, H]) -> logits [1, V] applies W_lm (kept
    fp16). Returns (logits of the last prompt token [V], residual rows [n, H])."""
    x = np.asarray(x0, dtype=np.float64)
    for lw, (kp, vp) in zip(layer_weights, pools):
        x = prefill_layer(x, lw, kp, vp, page_table_row, start, shape, exact, mirror)
    xf = od.rmsnorm(x[-1:], final_norm, shape.eps, exact)
    return lm_head_rows(xf)[0], x
