"""Materialise a synthetic workload on the GPU through the library's packers.

Used by the GPU tests and the benchmark (never by the oracle). Weights are
generated layer by layer, packed with pack_weights_w4g128 / pack_weights_f16
and copied into torch device tensors, so host memory stays bounded even for
the full 28-layer model.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np
import torch

import w4a16_paged_kv_amd as w4
from . import ROW_CHUNK, Workload, chunk_rows, embedding_chunk, lm_head_chunk, n_chunks


def to_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.float16)
    else:
        t = torch.from_numpy(a)
    return t.to(device)


def config_of(w: Workload) -> w4.w4_config:
    sh = w.shape
    return w4.make_config(sh.hidden, sh.n_heads, sh.n_kv_heads, sh.head_dim, sh.ffn, sh.vocab,
                          max(1, w.layers), sh.eps, sh.rope_base)


def upload_layer(w: Workload, l: int, bias: bool = False, device="cuda") -> Dict[str, torch.Tensor]:
    sh = w.shape
    lw = w.layer(l, bias=bias)
    d = {
        "qkv": to_dev(w4.pack_weights_w4g128(lw.qkv_q, lw.qkv_s, w4.ROLE_QKV, sh.head_dim), device),
        "o": to_dev(w4.pack_weights_w4g128(lw.o_q, lw.o_s), device),
        "gate_up": to_dev(w4.pack_weights_w4g128(lw.gate_up_q, lw.gate_up_s, w4.ROLE_GATE_UP), device),
        "down": to_dev(w4.pack_weights_w4g128(lw.down_q, lw.down_s), device),
        "attn_norm": to_dev(lw.attn_norm, device),
        "mlp_norm": to_dev(lw.mlp_norm, device),
    }
    if lw.qkv_bias is not None:
        d["qkv_bias"] = to_dev(lw.qkv_bias, device)
    return d


def k_pages_device(k: np.ndarray) -> np.ndarray:
    """K pages [..][16 tokens][D] in the device's slice order, same shape:
    value (t, d) at flat ((d // 32) * 64 + 16 ((d // 8) % 4) + t) * 8 + d % 8
    of its slice (the operand order of the attention's scores)."""
    *lead, T, D = k.shape
    n = len(lead)
    s = k.reshape(*lead, T, D // 32, 4, 8)             # t, d = 32P + 8c + e
    s = s.transpose(*range(n), n + 1, n + 2, n, n + 3)  # [P][c][t][e]
    return np.ascontiguousarray(s).reshape(*lead, T, D)


def k_pages_host(kd):
    """Inverse of k_pages_device (numpy arrays or torch tensors)."""
    *lead, T, D = kd.shape
    n = len(lead)
    s = kd.reshape(*lead, D // 32, 4, T, 8)             # [P][c][t][e]
    order = (*range(n), n + 2, n, n + 1, n + 3)         # -> [t][P][c][e]
    s = s.permute(*order) if hasattr(s, "permute") else s.transpose(*order)
    return s.reshape(*lead, T, D)


def v_pages_device(v: np.ndarray) -> np.ndarray:
    """V pages [..][16 tokens][D] in the device's slice order, same shape:
    value (t, d) at flat ((d // 32) * 64 + d % 16 + 16 (t // 4)) * 8 +
    ((d // 16) % 2) * 4 + t % 4 of its slice (the operand order of the
    attention's P V product)."""
    *lead, T, D = v.shape
    s = v.reshape(*lead, 4, 4, D // 32, 2, 16)          # t = 4q + j, d = 32P + 16e + r
    n = len(lead)
    s = s.transpose(*range(n), n + 2, n, n + 4, n + 3, n + 1)  # [P][q][r][e][j]
    return np.ascontiguousarray(s).reshape(*lead, T, D)


def v_pages_host(vd):
    """Inverse of v_pages_device (numpy arrays or torch tensors)."""
    *lead, T, D = vd.shape
    n = len(lead)
    s = vd.reshape(*lead, D // 32, 4, 16, 2, 4)         # [P][q][r][e][j]
    order = (*range(n), n + 1, n + 4, n, n + 3, n + 2)  # -> [q][j][P][e][r]
    s = s.permute(*order) if hasattr(s, "permute") else s.transpose(*order)
    return s.reshape(*lead, T, D)


def upload_kv(w: Workload, kv_cache: torch.Tensor, l: int, kv=None) -> None:
    """Copy layer l's generated K and V pages into the [L][2][P][Hkv][16 x D] cache
    (K and V slices in the device orders of k_pages_device and v_pages_device)."""
    k, v = kv if kv is not None else w.kv(l)
    kv_cache[l, 0].copy_(to_dev(k_pages_device(k), kv_cache.device).view(kv_cache[l, 0].shape))
    kv_cache[l, 1].copy_(to_dev(v_pages_device(v), kv_cache.device).view(kv_cache[l, 1].shape))


def upload_embedding(w: Workload, device="cuda") -> torch.Tensor:
    sh = w.shape
    e = torch.empty((sh.vocab, sh.hidden), dtype=torch.float16, device=device)
    for c in range(n_chunks(sh)):
        e[c * ROW_CHUNK: c * ROW_CHUNK + chunk_rows(sh, c)].copy_(to_dev(embedding_chunk(w.workload_id, sh, c), device))
    return e


def upload_lm_head(w: Workload, device="cuda") -> torch.Tensor:
    """Packed fp16 lm_head: chunks of 4096 rows are whole 16-row tiles, so the
    packed chunks concatenate into the packed matrix."""
    sh = w.shape
    buf = torch.empty(w4.w4_packed_f16_bytes(sh.vocab, sh.hidden), dtype=torch.uint8, device=device)
    off = 0
    for c in range(n_chunks(sh)):
        p = w4.pack_weights_f16(lm_head_chunk(w.workload_id, sh, c))
        buf[off:off + p.size].copy_(to_dev(p, device))
        off += p.size
    assert off == buf.numel()
    return buf


class DeviceModel:
    """A Workload's weights, KV cache and workspace on the GPU + its w4 Model."""

    def __init__(self, w: Workload, max_batch: Optional[int] = None, bias: bool = False,
                 device="cuda", progress=None, num_pages: Optional[int] = None):
        self.w = w
        self.cfg = config_of(w)
        nl = max(1, w.layers)
        self.num_pages = num_pages or w.num_pages
        self.max_batch = max_batch or w.batch
        self.max_pages = w.max_pages
        sh = w.shape
        self.layers = []
        self.kv_cache = torch.empty((nl, 2, self.num_pages, sh.n_kv_heads, 16, sh.head_dim),
                                    dtype=torch.float16, device=device)
        for l in range(nl):
            self.layers.append(upload_layer(w, l, bias, device))
            upload_kv(w, self.kv_cache, l)
            if progress:
                progress(l)
        self.embed = self.final_norm = self.lm_head = None
        if w.lm_head:
            self.embed = upload_embedding(w, device)
            self.final_norm = to_dev(w.final_norm(), device)
            self.lm_head = upload_lm_head(w, device)
        ws = w4.w4_workspace_bytes(self.cfg, self.max_batch, self.max_pages)
        assert ws > 0
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=device)
        self.model = w4.Model(self.cfg, self.layers, self.kv_cache, self.num_pages, self.workspace,
                              self.max_batch, self.max_pages, self.embed, self.final_norm, self.lm_head)

    def step_inputs(self):
        w = self.w
        return w.tokens(), w.positions, w.page_tables, w.ctx_lens
