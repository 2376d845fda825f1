"""Brute-force dense decode (test infrastructure only; see package header).

A second, independent statement of the same computation with none of the
paged machinery: weights are dense float64 matrices W = q * s expanded per
element with explicit loops over groups, the KV history is a contiguous
[ctx, D] array per KV head, and grouped-query attention is computed as plain
multi-head attention after repeating every KV head Hq / Hkv times. It is used
on tiny shapes to cross-check ``oracle.decode`` (exact mode, 1e-9).
"""
from __future__ import annotations

import math

import numpy as np


def dense_weight(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    n, k = q.shape
    w = np.zeros((n, k), dtype=np.float64)
    for g in range(s.shape[1]):
        lo, hi = 128 * g, min(k, 128 * g + 128)
        w[:, lo:hi] = q[:, lo:hi].astype(np.float64) * s[:, g:g + 1].astype(np.float64)
    return w


def rms(x, gamma, eps):
    return x / math.sqrt(sum(float(t) * float(t) for t in x) / len(x) + eps) * gamma


def rotate(v, pos, base):
    """RoPE as complex multiplication: z_i = v_i + i v_{i+D/2}, z_i <- z_i e^{i theta_i}."""
    d = v.shape[-1]
    half = d // 2
    z = v[..., :half] + 1j * v[..., half:]
    th = pos * base ** (-2.0 * np.arange(half) / d)
    z = z * np.exp(1j * th)
    return np.concatenate([z.real, z.imag], axis=-1)


def mha(q, k_hist, v_hist):
    """q [H, D]; k_hist/v_hist [H, T, D] (already repeated per q head)."""
    d = q.shape[-1]
    out = np.empty_like(q)
    for h in range(q.shape[0]):
        s = k_hist[h] @ q[h] / math.sqrt(d)
        p = np.exp(s - s.max())
        p = p / p.sum()
        out[h] = p @ v_hist[h]
    return out


def dense_layer(x, w, k_hist, v_hist, pos, shape):
    """One layer with a contiguous KV history. k_hist/v_hist: [Hkv, pos, D]
    (tokens before pos). Returns (x_out, k_new [Hkv, D], v_new [Hkv, D])."""
    sh = shape
    x = np.asarray(x, dtype=np.float64)
    xn = rms(x, w.attn_norm.astype(np.float64), sh.eps)
    y = dense_weight(w.qkv_q, w.qkv_s) @ xn
    if w.qkv_bias is not None:
        y = y + w.qkv_bias.astype(np.float64)
    nq, nkv = sh.q_rows, sh.kv_rows
    q = rotate(y[:nq].reshape(sh.n_heads, sh.head_dim), pos, sh.rope_base)
    k = rotate(y[nq:nq + nkv].reshape(sh.n_kv_heads, sh.head_dim), pos, sh.rope_base)
    v = y[nq + nkv:].reshape(sh.n_kv_heads, sh.head_dim)
    kh = np.concatenate([k_hist, k[:, None, :]], axis=1)
    vh = np.concatenate([v_hist, v[:, None, :]], axis=1)
    rep = sh.n_heads // sh.n_kv_heads
    o = mha(q, np.repeat(kh, rep, axis=0), np.repeat(vh, rep, axis=0))
    x1 = x + dense_weight(w.o_q, w.o_s) @ o.reshape(-1)
    xn2 = rms(x1, w.mlp_norm.astype(np.float64), sh.eps)
    g = dense_weight(w.gate_up_q[:sh.ffn], w.gate_up_s[:sh.ffn]) @ xn2
    u = dense_weight(w.gate_up_q[sh.ffn:], w.gate_up_s[sh.ffn:]) @ xn2
    h = g / (1.0 + np.exp(-g)) * u
    return x1 + dense_weight(w.down_q, w.down_s) @ h, k, v
