"""Paged W4A16 decode step in float64 (test infrastructure only; see package header).

Rounding: ``r`` is IEEE binary16 round-to-nearest-even; every other operation
is float64. With ``exact=True`` no rounding is applied anywhere (used to
compare against the dense brute force at 1e-9).

``mirror=True`` moves the rounding points: it also rounds the gate and up
projections before SiLU and q/k before RoPE. It is an equally plausible
fp16 reading of the pages, used only to measure how far two faithful
placements of the roundings drift apart over a whole layer or step (the
envelope a fused GPU computation is held to). Off by default.
"""
from __future__ import annotations

import numpy as np

PAGE = 16
GROUP = 128


def r16(x, exact: bool = False) -> np.ndarray:
    """Round to IEEE binary16 (nearest even) and return as float64."""
    x = np.asarray(x, dtype=np.float64)
    if exact:
        return x
    return x.astype(np.float16).astype(np.float64)


# ---------------------------------------------------------------- weights

def dequant_w4g128(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """W[n, k] = q[n, k] * s[n, k // 128] (symmetric, no zero point).

    Cite: "How to build your own LLM runtime from scratch", Architectural
    decisions and optimizations -- symmetric group-wise INT4 with group 128.
    Groups run along the input dimension k, one fp16 scale per row and group.
    The product is exact in float64.
    """
    q = np.asarray(q)
    assert q.dtype == np.int8 and q.min(initial=0) >= -8 and q.max(initial=0) <= 7
    n, k = q.shape
    ng = (k + GROUP - 1) // GROUP
    assert s.shape == (n, ng)
    sk = np.repeat(np.asarray(s, dtype=np.float64), GROUP, axis=1)[:, :k]
    return q.astype(np.float64) * sk


def gemv_w4(q: np.ndarray, s: np.ndarray, x: np.ndarray, rows_per_chunk: int = 4096) -> np.ndarray:
    """y[n] = sum_k W[n, k] x[k] with W = dequant_w4g128(q, s), in float64.
    x may carry leading batch dimensions ([..., K] -> [..., N]).

    The matrix is dequantised a band of rows at a time to bound memory; each
    output is still one full-length float64 dot product.
    """
    x = np.asarray(x, dtype=np.float64)
    lead = x.shape[:-1]
    xb = x.reshape(-1, x.shape[-1]).T                      # [K, B]
    n = q.shape[0]
    y = np.empty((n, xb.shape[1]), dtype=np.float64)
    for r0 in range(0, n, rows_per_chunk):
        r1 = min(n, r0 + rows_per_chunk)
        y[r0:r1] = dequant_w4g128(q[r0:r1], s[r0:r1]) @ xb
    return y.T.reshape(lead + (n,))


# ---------------------------------------------------------------- elementwise

def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float, exact: bool = False) -> np.ndarray:
    """y_i = r(x_i / sqrt(mean(x^2) + eps) * gamma_i), kept in FP16.

    Cite: "How to build your own LLM runtime from scratch", Architectural
    decisions and optimizations -- RMSNorm stays in FP16.
    """
    x = np.asarray(x, dtype=np.float64)
    ms = (x * x).sum(axis=-1, keepdims=True) / x.shape[-1]
    return r16(x / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64), exact)


def rope_angles(pos: int, head_dim: int, base: float) -> np.ndarray:
    """theta_i = pos * base^(-2 i / D) for i in [0, D/2)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return float(pos) * np.power(float(base), -2.0 * i / head_dim)


def rope(v: np.ndarray, pos: int, base: float, exact: bool = False) -> np.ndarray:
    """Rotate-half RoPE of one head vector v [D] (pairs i and i + D/2).

    v'_i       = v_i cos(theta_i) - v_{i+D/2} sin(theta_i)
    v'_{i+D/2} = v_{i+D/2} cos(theta_i) + v_i sin(theta_i)
    """
    v = np.asarray(v, dtype=np.float64)
    half = v.shape[-1] // 2
    th = rope_angles(pos, v.shape[-1], base)
    c, s = np.cos(th), np.sin(th)
    a, b = v[..., :half], v[..., half:]
    return r16(np.concatenate([a * c - b * s, b * c + a * s], axis=-1), exact)


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + e^-z)."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


# ---------------------------------------------------------------- paging

def page_slot(page_table_row: np.ndarray, t: int):
    """Logical token t lives in physical page page_table_row[t // 16], slot t % 16.

    Cite: "Building a Custom LLM Inference Runtime on H100", The Three
    Critical Bugs, Bug 1 (logical position -> physical block) and "How to
    build your own LLM runtime from scratch", Architectural decisions and
    optimizations (16-token pages).
    """
    return int(page_table_row[t // PAGE]), t % PAGE


def kv_write(k_pool: np.ndarray, v_pool: np.ndarray, page_table_row: np.ndarray, pos: int,
             k: np.ndarray, v: np.ndarray) -> None:
    """Store the new token's K and V (all KV heads) at its page slot, in place."""
    page, slot = page_slot(page_table_row, pos)
    k_pool[page, :, slot, :] = k
    v_pool[page, :, slot, :] = v


def gather_kv(pool: np.ndarray, page_table_row: np.ndarray, ctx: int, kv_head: int) -> np.ndarray:
    """Logical rows [ctx, D] of one KV head, read token by token through the page table."""
    rows = np.empty((ctx, pool.shape[-1]), dtype=np.float64)
    for t in range(ctx):
        page, slot = page_slot(page_table_row, t)
        rows[t] = pool[page, kv_head, slot, :]
    return rows


def softmax(s: np.ndarray) -> np.ndarray:
    """Max-subtracted softmax over the last axis."""
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def attention_decode(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                     page_table_row: np.ndarray, ctx: int, exact: bool = False) -> np.ndarray:
    """One sequence: o_h = r(sum_t softmax_t(q_h . K_t / sqrt(D)) V_t) for every q head.

    q: [Hq, D]; pools [P, Hkv, 16, D]. q head h reads KV head h // (Hq / Hkv)
    (GQA 7:1 in the shapes used here). Only tokens [0, ctx) are read.
    Cite: "How to build your own LLM runtime from scratch", Architectural
    decisions and optimizations (GQA 7:1, 16-token pages); "Building a Custom
    LLM Inference Runtime on H100", The KV Cache and PagedAttention.
    """
    q = np.asarray(q, dtype=np.float64)
    hq, d = q.shape
    hkv = k_pool.shape[1]
    grp = hq // hkv
    out = np.empty((hq, d), dtype=np.float64)
    for j in range(hkv):
        kj = gather_kv(k_pool, page_table_row, ctx, j)
        vj = gather_kv(v_pool, page_table_row, ctx, j)
        for h in range(j * grp, (j + 1) * grp):
            p = softmax(kj @ q[h] / np.sqrt(d))
            out[h] = p @ vj
    return r16(out, exact)


def attention_partial(q: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray):
    """Un-normalised softmax state of one block of tokens for one head:
    m = max_t s_t, l = sum_t e^(s_t - m), o = sum_t e^(s_t - m) V_t."""
    s = k_rows @ np.asarray(q, dtype=np.float64) / np.sqrt(q.shape[-1])
    m = s.max()
    e = np.exp(s - m)
    return m, e.sum(), e @ v_rows


def lse_merge(parts) -> np.ndarray:
    """Combine per-block softmax states: with M = max m_s,
    o = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s (log-sum-exp merge)."""
    mm = max(m for m, _, _ in parts)
    num = sum(np.exp(m - mm) * o for m, _, o in parts)
    den = sum(np.exp(m - mm) * l for m, l, _ in parts)
    return num / den


# ---------------------------------------------------------------- layers

def qkv_stage(x: np.ndarray, w, pos: int, shape, exact: bool = False, mirror: bool = False):
    """xn = rmsnorm(x, gamma_attn); then qkv_from_normed(xn)."""
    xn = rmsnorm(np.asarray(x, dtype=np.float64), w.attn_norm, shape.eps, exact)
    return qkv_from_normed(xn, w, pos, shape, exact, mirror)


def qkv_from_normed(xn: np.ndarray, w, pos: int, shape, exact: bool = False, mirror: bool = False):
    """[q; k; v] = W_qkv xn (+ bias); returns (r(RoPE(q)) [Hq, D],
    r(RoPE(k)) [Hkv, D], r(v) [Hkv, D]) at position pos. q and k are rotated
    unrounded and rounded once afterwards (mirror: also rounded before)."""
    sh = shape
    xn = np.asarray(xn, dtype=np.float64)
    if xn.ndim == 2:   # a batch: one position per row
        y_all = gemv_w4(w.qkv_q, w.qkv_s, xn)
        outs = [_split_qkv(y_all[b], w, int(np.asarray(pos)[b]), sh, exact, mirror)
                for b in range(xn.shape[0])]
        return tuple(np.stack(t) for t in zip(*outs))
    return _split_qkv(gemv_w4(w.qkv_q, w.qkv_s, xn), w, pos, sh, exact, mirror)


def _split_qkv(y, w, pos, sh, exact, mirror=False):
    if w.qkv_bias is not None:
        y = y + np.asarray(w.qkv_bias, dtype=np.float64)
    nq, nkv = sh.q_rows, sh.kv_rows
    q = y[:nq].reshape(sh.n_heads, sh.head_dim)
    k = y[nq:nq + nkv].reshape(sh.n_kv_heads, sh.head_dim)
    v = r16(y[nq + nkv:].reshape(sh.n_kv_heads, sh.head_dim), exact)
    if mirror:
        q, k = r16(q, exact), r16(k, exact)
    return rope(q, pos, sh.rope_base, exact), rope(k, pos, sh.rope_base, exact), v


def oproj_stage(x: np.ndarray, o: np.ndarray, w, exact: bool = False) -> np.ndarray:
    """x1 = r(x + W_o o), o the concatenated attention heads [..., Hq D]."""
    x = np.asarray(x, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64).reshape(x.shape[:-1] + (-1,))
    return r16(x + gemv_w4(w.o_q, w.o_s, o), exact)


def gate_up_stage(x1: np.ndarray, w, shape, exact: bool = False, mirror: bool = False) -> np.ndarray:
    """xn2 = rmsnorm(x1, gamma_mlp); then gate_up_from_normed(xn2)."""
    xn2 = rmsnorm(np.asarray(x1, dtype=np.float64), w.mlp_norm, shape.eps, exact)
    return gate_up_from_normed(xn2, w, shape, exact, mirror)


def gate_up_from_normed(xn2: np.ndarray, w, shape, exact: bool = False, mirror: bool = False) -> np.ndarray:
    """h = r(silu(W_gate xn2) * (W_up xn2)); g and u unrounded (mirror: rounded)."""
    gu = gemv_w4(w.gate_up_q, w.gate_up_s, np.asarray(xn2, dtype=np.float64))
    g, u = gu[..., :shape.ffn], gu[..., shape.ffn:]
    if mirror:
        g, u = r16(g, exact), r16(u, exact)
    return r16(silu(g) * u, exact)


def down_stage(x1: np.ndarray, h: np.ndarray, w, exact: bool = False) -> np.ndarray:
    """x2 = r(x1 + W_down h)."""
    return r16(np.asarray(x1, dtype=np.float64) + gemv_w4(w.down_q, w.down_s, np.asarray(h, dtype=np.float64)),
               exact)


def decode_layer(x: np.ndarray, w, k_pool: np.ndarray, v_pool: np.ndarray,
                 page_table_row: np.ndarray, ctx: int, shape, exact: bool = False,
                 mirror: bool = False) -> np.ndarray:
    """One decoder layer for one sequence; returns the new residual x [H] and
    updates the (float64) pools in place with the token's K and V.

    Steps (one rounding per stored tensor):
      xn = rmsnorm(x, gamma_attn)
      [q; k; v] = W_qkv xn (+ bias); v = r(v); q, k unrounded
      q', k' = r(RoPE(q)), r(RoPE(k)) at position pos = ctx - 1
      K/V pool slot of pos <- k', v  (before attention)
      o = attention over tokens [0, ctx)
      x1 = r(x + W_o o)
      xn2 = rmsnorm(x1, gamma_mlp)
      h = r(silu(W_gate xn2) * (W_up xn2))
      return r(x1 + W_down h)
    (mirror: g, u and the pre-RoPE q, k rounded too)
    """
    pos = ctx - 1
    q, k, v = qkv_stage(x, w, pos, shape, exact, mirror)
    kv_write(k_pool, v_pool, page_table_row, pos, k, v)
    o = attention_decode(q, k_pool, v_pool, page_table_row, ctx, exact)
    x1 = oproj_stage(x, o, w, exact)
    h = gate_up_stage(x1, w, shape, exact, mirror)
    return down_stage(x1, h, w, exact)


def lm_head(x: np.ndarray, final_norm: np.ndarray, w_lm: np.ndarray, eps: float,
            exact: bool = False) -> np.ndarray:
    """logits = r(W_lm rmsnorm(x, gamma_final)); W_lm is fp16, kept in FP16.

    Cite: "How to build your own LLM runtime from scratch", Architectural
    decisions and optimizations (lm_head stays in FP16).
    """
    xf = rmsnorm(x, final_norm, eps, exact)
    return r16(np.asarray(w_lm, dtype=np.float64) @ xf, exact)
