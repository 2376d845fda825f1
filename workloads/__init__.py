"""Seeded synthetic inputs for the W4A16 paged-KV decode step.

This module only *draws* inputs. It holds none of the decode arithmetic: no
dequantisation, normalisation, rotation, attention or page addressing. Both
the oracle and the GPU path read what it returns.

Every tensor comes from its own stream,
``numpy.random.default_rng(SeedSequence([workload_id, layer, tensor_id, chunk]))``,
so any tensor (or row chunk of a large one) can be regenerated on its own.

Distributions (one reading of the workload descriptions):
  * INT4 weights: q uniform over the integers [-8, 7]; one fp16 scale per row
    and per 128 consecutive input columns, s = fp16(0.02 * |N(0, 1)|).
  * Activations, embedding rows, KV cache contents, attention queries:
    fp16(N(0, 1)).
  * RMSNorm weights gamma = 1.0 (``gamma="ones"``) or fp16(1 + 0.1 N(0, 1))
    (``gamma="random"``, used by unit tests to expose indexing mistakes).
  * fp16 lm_head: fp16(q * s) with q and s drawn as for the INT4 weights.
  * Context lengths: integers uniform over [lo, hi] inclusive; the page pool
    holds exactly sum(ceil(ctx / 16)) pages, dealt out by one random
    permutation in sequence order. Page tables are -1 padded.
  * Token ids: uniform over [0, vocab).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Dict, List, Optional, Tuple

import numpy as np

PAGE = 16      # tokens per KV page
GROUP = 128    # input columns per INT4 scale group

# tensor ids of the seed streams
QKV, O, GATE_UP, DOWN = 0, 1, 2, 3
ATTN_NORM, MLP_NORM = 4, 5
K_CACHE, V_CACHE = 6, 7
X_IN, PAGE_TABLE, CTX, TOKENS = 8, 9, 10, 11
EMBED, LM_HEAD, FINAL_NORM = 12, 13, 14
Q_ATTN, QKV_BIAS = 15, 16
FORCED_ROW = 17
PROMPT = 18

ROW_CHUNK = 4096   # row chunk of the per-chunk streams (embedding, lm_head)


@dataclass(frozen=True)
class Shape:
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    n_layers: int
    eps: float = 1e-6
    rope_base: float = 1e6

    @property
    def q_rows(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_rows(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def qkv_rows(self) -> int:
        return self.q_rows + 2 * self.kv_rows

    @property
    def group_size(self) -> int:
        return self.n_heads // self.n_kv_heads


# Qwen2.5-7B decoder shape and its one-layer miniature (GQA 7:1 in both).
QWEN7B = Shape(hidden=3584, n_heads=28, n_kv_heads=4, head_dim=128, ffn=18944,
               vocab=152064, n_layers=28)
MINI = Shape(hidden=448, n_heads=7, n_kv_heads=1, head_dim=64, ffn=1536,
             vocab=4096, n_layers=1)


def rng(workload_id: int, layer: int, tensor_id: int, chunk: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([workload_id, layer, tensor_id, chunk]))


def f16_normal(g: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    return (g.standard_normal(shape, dtype=np.float32) * np.float32(scale)).astype(np.float16)


def int4_uniform(g: np.random.Generator, n: int, k: int) -> np.ndarray:
    """q[n, k] uniform over {-8..7} (int8). Each random byte supplies two values."""
    assert k % 2 == 0
    b = np.frombuffer(g.bytes(n * k // 2), dtype=np.uint8).reshape(n, k // 2)
    q = np.empty((n, k), dtype=np.int8)
    q[:, 0::2] = (b & 15).astype(np.int8) - 8
    q[:, 1::2] = (b >> 4).astype(np.int8) - 8
    return q


def group_scales(g: np.random.Generator, n: int, k: int) -> np.ndarray:
    ng = (k + GROUP - 1) // GROUP
    return np.abs(g.standard_normal((n, ng), dtype=np.float32) * np.float32(0.02)).astype(np.float16)


def int4_matrix(workload_id: int, layer: int, tensor_id: int, n: int, k: int,
                chunk: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """(q int8 [n, k] in [-8, 7], s fp16 [n, ceil(k/128)])."""
    g = rng(workload_id, layer, tensor_id, chunk)
    q = int4_uniform(g, n, k)
    s = group_scales(g, n, k)
    return q, s


def norm_weight(workload_id: int, layer: int, tensor_id: int, n: int, gamma: str) -> np.ndarray:
    if gamma == "ones":
        return np.ones(n, dtype=np.float16)
    g = rng(workload_id, layer, tensor_id)
    return (1.0 + 0.1 * g.standard_normal(n, dtype=np.float32)).astype(np.float16)


@dataclass
class LayerWeights:
    qkv_q: np.ndarray      # int8 [(Hq + 2 Hkv) D, H]: q heads, then k heads, then v heads
    qkv_s: np.ndarray
    o_q: np.ndarray        # int8 [H, Hq D]
    o_s: np.ndarray
    gate_up_q: np.ndarray  # int8 [2F, H]: gate rows [0, F), up rows [F, 2F)
    gate_up_s: np.ndarray
    down_q: np.ndarray     # int8 [H, F]
    down_s: np.ndarray
    attn_norm: np.ndarray  # fp16 [H]
    mlp_norm: np.ndarray   # fp16 [H]
    qkv_bias: Optional[np.ndarray] = None   # fp16 [(Hq + 2 Hkv) D] or None


def layer_weights(workload_id: int, layer: int, sh: Shape, gamma: str = "ones",
                  bias: bool = False) -> LayerWeights:
    qkv_q, qkv_s = int4_matrix(workload_id, layer, QKV, sh.qkv_rows, sh.hidden)
    o_q, o_s = int4_matrix(workload_id, layer, O, sh.hidden, sh.q_rows)
    gu_q, gu_s = int4_matrix(workload_id, layer, GATE_UP, 2 * sh.ffn, sh.hidden)
    d_q, d_s = int4_matrix(workload_id, layer, DOWN, sh.hidden, sh.ffn)
    b = None
    if bias:
        b = f16_normal(rng(workload_id, layer, QKV_BIAS), sh.qkv_rows, 0.5)
    return LayerWeights(qkv_q, qkv_s, o_q, o_s, gu_q, gu_s, d_q, d_s,
                        norm_weight(workload_id, layer, ATTN_NORM, sh.hidden, gamma),
                        norm_weight(workload_id, layer, MLP_NORM, sh.hidden, gamma), b)


def embedding_rows(workload_id: int, sh: Shape, rows: np.ndarray) -> np.ndarray:
    """Rows of the fp16 N(0,1) embedding table [vocab, H], drawn per 4096-row chunk."""
    out = np.empty((len(rows), sh.hidden), dtype=np.float16)
    for c in np.unique(np.asarray(rows) // ROW_CHUNK):
        blk = embedding_chunk(workload_id, sh, int(c))
        sel = np.nonzero(np.asarray(rows) // ROW_CHUNK == c)[0]
        out[sel] = blk[np.asarray(rows)[sel] - c * ROW_CHUNK]
    return out


def n_chunks(sh: Shape) -> int:
    return (sh.vocab + ROW_CHUNK - 1) // ROW_CHUNK


def chunk_rows(sh: Shape, c: int) -> int:
    return min(ROW_CHUNK, sh.vocab - c * ROW_CHUNK)


def embedding_chunk(workload_id: int, sh: Shape, c: int) -> np.ndarray:
    return f16_normal(rng(workload_id, 0, EMBED, c), (chunk_rows(sh, c), sh.hidden))


def lm_head_chunk(workload_id: int, sh: Shape, c: int) -> np.ndarray:
    """Rows [4096 c, 4096 c + 4096) of the fp16 lm_head [vocab, H] = fp16(q * s)."""
    n = chunk_rows(sh, c)
    q, s = int4_matrix(workload_id, 0, LM_HEAD, n, sh.hidden, chunk=c)
    ss = np.repeat(s.astype(np.float32), GROUP, axis=1)[:, :sh.hidden]
    return (q.astype(np.float32) * ss).astype(np.float16)   # q*s is exact in fp32


def kv_pages(workload_id: int, layer: int, sh: Shape, num_pages: int) -> Tuple[np.ndarray, np.ndarray]:
    """Physical K and V pools of one layer, fp16 [P, Hkv, 16, D], every slot N(0,1)."""
    shp = (num_pages, sh.n_kv_heads, PAGE, sh.head_dim)
    return (f16_normal(rng(workload_id, layer, K_CACHE), shp),
            f16_normal(rng(workload_id, layer, V_CACHE), shp))


def deal_pages(workload_id: int, ctx_lens: np.ndarray) -> Tuple[np.ndarray, int]:
    """Page tables [B, max_pages] (-1 padded) dealt from one permuted pool."""
    need = (np.asarray(ctx_lens) + PAGE - 1) // PAGE
    total = int(need.sum())
    perm = rng(workload_id, 0, PAGE_TABLE).permutation(total).astype(np.int32)
    max_pages = int(need.max())
    pt = np.full((len(ctx_lens), max_pages), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(need):
        pt[b, :n] = perm[off:off + n]
        off += n
    return pt, total


@dataclass
class Workload:
    """One synthetic decode workload: shapes, batch state and seed id."""
    name: str
    workload_id: int
    shape: Shape
    batch: int
    ctx_lens: np.ndarray     # int32 [B], counts the token being decoded
    page_tables: np.ndarray  # int32 [B, max_pages], -1 padded
    num_pages: int
    layers: int              # decoder layers run by this workload
    lm_head: bool            # full step (embedding + layers + final norm + lm_head)
    gamma: str = "ones"

    @property
    def positions(self) -> np.ndarray:
        return (self.ctx_lens - 1).astype(np.int32)

    @property
    def max_pages(self) -> int:
        return self.page_tables.shape[1]

    def tokens(self) -> np.ndarray:
        return rng(self.workload_id, 0, TOKENS).integers(0, self.shape.vocab, self.batch).astype(np.int32)

    def prompt_tokens(self, n: int) -> np.ndarray:
        """Prompt token ids for prefill: n ids uniform over [0, vocab)."""
        return rng(self.workload_id, 0, PROMPT).integers(0, self.shape.vocab, n).astype(np.int32)

    def x_in(self) -> np.ndarray:
        """Layer input activations fp16 [B, H] (single-layer workloads)."""
        return f16_normal(rng(self.workload_id, 0, X_IN), (self.batch, self.shape.hidden))

    def layer(self, l: int, bias: bool = False) -> LayerWeights:
        return layer_weights(self.workload_id, l, self.shape, self.gamma, bias)

    def kv(self, l: int) -> Tuple[np.ndarray, np.ndarray]:
        return kv_pages(self.workload_id, l, self.shape, self.num_pages)

    def final_norm(self) -> np.ndarray:
        return norm_weight(self.workload_id, 0, FINAL_NORM, self.shape.hidden, self.gamma)

    def attn_q(self) -> np.ndarray:
        """Attention-only workloads: queries fp16 [B, Hq, D]."""
        sh = self.shape
        return f16_normal(rng(self.workload_id, 0, Q_ATTN), (self.batch, sh.n_heads, sh.head_dim))


def forced_rows(workload_id: int, layer: int, rows, hidden: int) -> np.ndarray:
    """Finite stand-in residual rows fp16 N(0, 1) [len(rows), hidden], one
    stream per (layer, row): fed to a layer in place of a sequence whose
    residual stream has overflowed fp16, so that layer can still be compared
    for that sequence (rows are independent of each other)."""
    return np.stack([f16_normal(rng(workload_id, layer, FORCED_ROW, int(b)), hidden) for b in rows]) \
        if len(rows) else np.zeros((0, hidden), np.float16)


def _make(name, wid, shape, ctx_lens, layers, lm_head, gamma="ones") -> Workload:
    ctx = np.asarray(ctx_lens, dtype=np.int32)
    pt, total = deal_pages(wid, ctx)
    return Workload(name, wid, shape, len(ctx), ctx, pt, total, layers, lm_head, gamma)


def _uniform_ctx(wid: int, batch: int, lo: int, hi: int) -> np.ndarray:
    return rng(wid, 0, CTX).integers(lo, hi + 1, batch).astype(np.int32)


def layer_mini() -> Workload:
    """One decoder layer of the miniature (hidden 448, 7 q heads : 1 kv head,
    head_dim 64, FFN 1536), batch 1, 64 context tokens in 4 shuffled pages."""
    return _make("layer_mini", 0, MINI, [64], 1, False)


def layer_full() -> Workload:
    """One decoder layer at the Qwen2.5-7B shape, batch 1, 512 tokens (32 pages)."""
    return _make("layer_full", 1, QWEN7B, [512], 1, False)


def step_b1() -> Workload:
    """Full 28-layer step + final norm + fp16 lm_head, batch 1, 2048 tokens."""
    return _make("step_b1", 2, QWEN7B, [2048], QWEN7B.n_layers, True)


def attn_stress() -> Workload:
    """Paged attention only: 32 sequences, contexts uniform over [128, 8192]."""
    return _make("attn_stress", 3, QWEN7B, _uniform_ctx(3, 32, 128, 8192), 0, False)


def step_b16() -> Workload:
    """Full 28-layer step, batch 16, contexts uniform over [1024, 4096]."""
    return _make("step_b16", 4, QWEN7B, _uniform_ctx(4, 16, 1024, 4096), QWEN7B.n_layers, True)


def prefill_512() -> Workload:
    """Prefill of a 512-token prompt (positions 0..511, 32 shuffled pages) through
    the full 28-layer model + final norm + lm_head of the last token."""
    return _make("prefill_512", 5, QWEN7B, [512], QWEN7B.n_layers, True)


WORKLOADS = {"layer_mini": layer_mini, "layer_full": layer_full, "step_b1": step_b1,
             "attn_stress": attn_stress, "step_b16": step_b16, "prefill_512": prefill_512}


def custom(name: str, wid: int, shape: Shape, ctx_lens, layers: int = 1, lm_head: bool = False,
           gamma: str = "ones") -> Workload:
    """Small ad-hoc workloads for unit tests (any shape, any context lengths)."""
    return _make(name, wid, shape, ctx_lens, layers, lm_head, gamma)

