"""Python binding of libw4a16 (ctypes): the single-token decode step of a
GQA transformer with W4A16 projections and a paged fp16 KV cache, on
MI355X (gfx950).

Argument marshalling only. Every step of the decode path runs in the
library's HIP kernels; PyTorch supplies device memory and streams. The
functions keep the C names of include/w4a16.h. If the library is missing the
import still succeeds, but the first call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_float, c_int, c_int32, c_int64, c_size_t, c_uint32, c_void_p
from typing import List, Optional, Sequence

import numpy as np

# W4A16_LIB selects another build of the same library (the host-sanitizer
# build the CPU tests run under); by default the in-tree libw4a16.so.
LIB_PATH = os.environ.get("W4A16_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libw4a16.so")

W4_OK, W4_EINVAL, W4_ERANGE, W4_EALIGN, W4_ENOPAGES, W4_EHIP, W4_ESTATE = range(7)
ERROR_NAMES = {1: "EINVAL", 2: "ERANGE", 3: "EALIGN", 4: "ENOPAGES", 5: "EHIP", 6: "ESTATE"}
ROLE_PLAIN, ROLE_QKV, ROLE_GATE_UP = 0, 1, 2
OP_EMBED, OP_QKV, OP_ATTN, OP_OPROJ, OP_GATE_UP, OP_DOWN, OP_LM_HEAD = range(7)
BUF_X, BUF_Q, BUF_O, BUF_H, BUF_XN = range(5)
PAGE = 16


class W4Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"W4_{ERROR_NAMES.get(code, code)}: {msg}")
        self.code = code


class w4_config(Structure):
    _fields_ = [("hidden", c_int32), ("n_heads", c_int32), ("n_kv_heads", c_int32),
                ("head_dim", c_int32), ("ffn", c_int32), ("vocab", c_int32),
                ("n_layers", c_int32), ("rms_eps", c_float), ("rope_base", c_float)]


class w4_layer_weights(Structure):
    _fields_ = [("qkv", c_void_p), ("o", c_void_p), ("gate_up", c_void_p), ("down", c_void_p),
                ("attn_norm", c_void_p), ("mlp_norm", c_void_p), ("qkv_bias", c_void_p)]


class w4_weights(Structure):
    _fields_ = [("layers", POINTER(w4_layer_weights)), ("embed", c_void_p),
                ("final_norm", c_void_p), ("lm_head", c_void_p)]


_SIGS = {
    "w4_last_error": (ctypes.c_char_p, []),
    "w4_version": (ctypes.c_char_p, []),
    "w4_packed_bytes": (c_size_t, [c_int32, c_int32]),
    "pack_weights_w4g128": (c_int, [c_void_p, c_void_p, c_int32, c_int32, c_uint32, c_int32, c_void_p, c_size_t]),
    "quantize_w4g128": (c_int, [c_void_p, c_int32, c_int32, c_void_p, c_void_p]),
    "w4_packed_f16_bytes": (c_size_t, [c_int32, c_int32]),
    "pack_weights_f16": (c_int, [c_void_p, c_int32, c_int32, c_void_p, c_size_t]),
    "kv_pool_create": (c_int, [c_int32, c_int32, POINTER(c_void_p)]),
    "kv_pool_destroy": (None, [c_void_p]),
    "kv_alloc_pages": (c_int, [c_void_p, c_int32, c_void_p]),
    "kv_free_pages": (c_int, [c_void_p, c_void_p, c_int32]),
    "kv_free_count": (c_int32, [c_void_p]),
    "kv_seq_reserve": (c_int, [c_void_p, c_int32, c_int32]),
    "kv_seq_release": (c_int, [c_void_p, c_int32]),
    "kv_seq_pages": (c_int32, [c_void_p, c_int32]),
    "page_table": (c_int, [c_void_p, c_void_p, c_int32, c_int32, c_void_p]),
    "kv_cache_bytes": (c_size_t, [POINTER(w4_config), c_int32]),
    "w4_workspace_bytes": (c_size_t, [POINTER(w4_config), c_int32, c_int32]),
    "w4_model_create": (c_int, [POINTER(w4_config), POINTER(w4_weights), c_void_p, c_int32, c_void_p,
                                c_size_t, c_int32, c_int32, POINTER(c_void_p)]),
    "w4_model_destroy": (None, [c_void_p]),
    "w4_set_graph": (c_int, [c_void_p, c_int]),
    "decode_step": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p]),
    "decode_step_device": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p]),
    "w4_device_errors": (c_int64, [c_void_p, c_void_p]),
    "w4_validate_step": (c_int, [POINTER(w4_config), c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_int32]),
    "w4_model_stage": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p]),
    "w4_model_run_op": (c_int, [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p]),
    "w4_model_buffer": (c_void_p, [c_void_p, c_int32, POINTER(c_int32)]),
    "decode_layer": (c_int, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p]),
    "w4_gemv": (c_int, [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_void_p]),
    "w4_gemv_f16": (c_int, [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_void_p]),
    "paged_attention_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32, c_int32, c_int32]),
    "paged_attention_decode": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32,
                                       c_int32, c_int32, c_int32, c_int32, c_void_p, c_size_t, c_void_p, c_void_p]),
    "w4_prefill_workspace_bytes": (c_size_t, [POINTER(w4_config), c_int32, c_int32]),
    "w4_gemv_variant": (c_int, [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p]),
    "w4_prefill_buffer": (c_int64, [POINTER(w4_config), c_int32, c_int32, c_int32, POINTER(c_int32)]),
    "w4_prefill": (c_int, [c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_size_t, c_void_p, c_void_p]),
    "kv_write_pages": (c_int, [POINTER(w4_config), c_void_p, c_int32, c_int32, c_void_p, c_int32, c_int32, c_int32,
                               c_void_p, c_void_p, c_void_p]),
    "kv_read_pages": (c_int, [POINTER(w4_config), c_void_p, c_int32, c_int32, c_void_p, c_int32, c_int32, c_int32,
                              c_void_p, c_void_p, c_void_p]),
    "paged_attention_noalloc_max_bytes": (c_size_t, []),
    "paged_attention_decode_noalloc": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                               c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p]),
    "w4_argmax_workspace_bytes": (c_size_t, [c_int32, c_int32]),
    "w4_argmax_f16": (c_int, [c_void_p, c_int32, c_int32, c_void_p, c_size_t, c_void_p, c_void_p]),
    "w4_generate_greedy": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32,
                                   c_void_p, c_void_p, c_void_p, POINTER(c_int32), c_void_p]),
}
EXPORTED = sorted(_SIGS)

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m w4a16_paged_kv_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def _check(rc: int) -> None:
    if rc != W4_OK:
        raise W4Error(rc, lib().w4_last_error().decode())


def _ptr(a) -> Optional[int]:
    """Address of a numpy array, torch tensor or raw int (None -> NULL)."""
    if a is None:
        return None
    if isinstance(a, int):
        return a
    if isinstance(a, np.ndarray):
        assert a.flags["C_CONTIGUOUS"]
        return a.ctypes.data
    assert a.is_contiguous()
    return a.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def w4_version() -> str:
    return lib().w4_version().decode()


# ------------------------------------------------------------------ packing

def w4_packed_bytes(n: int, k: int) -> int:
    return lib().w4_packed_bytes(n, k)


def pack_weights_w4g128(q: np.ndarray, scales: np.ndarray, role: int = ROLE_PLAIN,
                        head_dim: int = 0) -> np.ndarray:
    """Pack int8 q [n, k] in [-8, 7] and fp16 scales [n, ceil(k/128)] -> uint8 buffer."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    scales = np.ascontiguousarray(scales, dtype=np.float16)
    n, k = q.shape
    out = np.empty(w4_packed_bytes(n, k), dtype=np.uint8)
    _check(lib().pack_weights_w4g128(_ptr(q), _ptr(scales), n, k, role, head_dim, _ptr(out), out.size))
    return out


def quantize_w4g128(w: np.ndarray):
    """fp16 [n, k] -> (q int8 [n, k], scales fp16 [n, ceil(k/128)]), host arrays."""
    w = np.ascontiguousarray(w, dtype=np.float16)
    n, k = w.shape
    q = np.empty((n, k), dtype=np.int8)
    s = np.empty((n, (k + 127) // 128), dtype=np.float16)
    _check(lib().quantize_w4g128(_ptr(w), n, k, _ptr(q), _ptr(s)))
    return q, s


def w4_packed_f16_bytes(n: int, k: int) -> int:
    return lib().w4_packed_f16_bytes(n, k)


def pack_weights_f16(w: np.ndarray) -> np.ndarray:
    w = np.ascontiguousarray(w, dtype=np.float16)
    n, k = w.shape
    out = np.empty(w4_packed_f16_bytes(n, k), dtype=np.uint8)
    _check(lib().pack_weights_f16(_ptr(w), n, k, _ptr(out), out.size))
    return out


# ------------------------------------------------------------------ KV pool

class KvPool:
    """Host page pool (kv_pool_*): free-list allocation, sequence page lists, page tables."""

    def __init__(self, num_pages: int, max_seqs: int):
        self.handle = None
        h = c_void_p()
        _check(lib().kv_pool_create(num_pages, max_seqs, ctypes.byref(h)))
        self.handle = h.value

    def close(self):
        if getattr(self, "handle", None):
            lib().kv_pool_destroy(self.handle)
            self.handle = None

    __del__ = close

    def kv_alloc_pages(self, n: int) -> np.ndarray:
        ids = np.empty(max(n, 1), dtype=np.int32)
        _check(lib().kv_alloc_pages(self.handle, n, _ptr(ids)))
        return ids[:n]

    def kv_free_pages(self, ids) -> None:
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        _check(lib().kv_free_pages(self.handle, _ptr(ids) if ids.size else None, ids.size))

    def kv_free_count(self) -> int:
        return lib().kv_free_count(self.handle)

    def kv_seq_reserve(self, seq: int, ctx_len: int) -> None:
        _check(lib().kv_seq_reserve(self.handle, seq, ctx_len))

    def kv_seq_release(self, seq: int) -> None:
        _check(lib().kv_seq_release(self.handle, seq))

    def kv_seq_pages(self, seq: int) -> int:
        return lib().kv_seq_pages(self.handle, seq)

    def page_table(self, seqs: Sequence[int], max_pages: int) -> np.ndarray:
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        out = np.empty((len(seqs), max_pages), dtype=np.int32)
        _check(lib().page_table(self.handle, _ptr(seqs), len(seqs), max_pages, _ptr(out)))
        return out


# ------------------------------------------------------------------ model

def make_config(hidden, n_heads, n_kv_heads, head_dim, ffn, vocab, n_layers, rms_eps=1e-6,
                rope_base=1e6) -> w4_config:
    return w4_config(hidden, n_heads, n_kv_heads, head_dim, ffn, vocab, n_layers, rms_eps, rope_base)


def kv_cache_bytes(cfg: w4_config, num_pages: int) -> int:
    return lib().kv_cache_bytes(ctypes.byref(cfg), num_pages)


def w4_workspace_bytes(cfg: w4_config, max_batch: int, max_pages: int) -> int:
    return lib().w4_workspace_bytes(ctypes.byref(cfg), max_batch, max_pages)


def w4_validate_step(cfg: w4_config, num_pages: int, max_batch: int, max_pages: int, tokens, positions,
                     page_tables, ctx_lens) -> None:
    arrs = [None if a is None else np.ascontiguousarray(a, dtype=np.int32)
            for a in (tokens, positions, page_tables, ctx_lens)]
    _check(lib().w4_validate_step(ctypes.byref(cfg), num_pages, max_batch, max_pages,
                                  *(_ptr(a) for a in arrs), len(arrs[1])))


class Model:
    """w4_model handle bound to caller-owned device tensors.

    layers: list of dicts with device tensors under the keys qkv, o, gate_up,
    down (packed), attn_norm, mlp_norm and optionally qkv_bias. The tensors
    are referenced (not copied) and kept alive by this object.
    """

    def __init__(self, cfg: w4_config, layers: List[dict], kv_cache, num_pages: int, workspace,
                 max_batch: int, max_pages: int, embed=None, final_norm=None, lm_head=None):
        self.cfg = cfg
        self._keep = [layers, kv_cache, workspace, embed, final_norm, lm_head]
        arr = (w4_layer_weights * len(layers))()
        for i, d in enumerate(layers):
            arr[i] = w4_layer_weights(_ptr(d["qkv"]), _ptr(d["o"]), _ptr(d["gate_up"]), _ptr(d["down"]),
                                      _ptr(d["attn_norm"]), _ptr(d["mlp_norm"]), _ptr(d.get("qkv_bias")))
        w = w4_weights(arr, _ptr(embed), _ptr(final_norm), _ptr(lm_head))
        self._arr = arr
        h = c_void_p()
        _check(lib().w4_model_create(ctypes.byref(cfg), ctypes.byref(w), _ptr(kv_cache), num_pages,
                                     _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     max_batch, max_pages, ctypes.byref(h)))
        self.handle = h.value
        self._destroy = lib().w4_model_destroy  # held: module globals may be gone when __del__ runs at exit
        self.kv_cache, self.workspace = kv_cache, workspace
        self.num_pages, self.max_batch, self.max_pages = num_pages, max_batch, max_pages

    def close(self):
        if getattr(self, "handle", None):
            self._destroy(self.handle)
            self.handle = None

    __del__ = close

    def w4_prefill(self, tokens, start: int, page_table, workspace, logits, stream=None) -> None:
        """Prompt tokens (host int32 [n]) at positions start.. through the model;
        page_table: host int32 [max_pages]; logits: device fp16 [vocab] of the
        last prompt token; workspace: device bytes >= w4_prefill_workspace_bytes."""
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        pt = np.ascontiguousarray(page_table, dtype=np.int32).reshape(-1)
        if pt.size != self.max_pages:
            raise ValueError(f"page_table has {pt.size} entries, the model {self.max_pages}")
        _check(lib().w4_prefill(self.handle, _ptr(t), t.size, start, _ptr(pt), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _ptr(logits), _stream(stream)))

    def w4_set_graph(self, enabled: bool) -> None:
        _check(lib().w4_set_graph(self.handle, int(enabled)))

    def decode_step(self, tokens, positions, page_tables, ctx_lens, logits, stream=None) -> None:
        """Host int32 arrays (tokens/positions/ctx_lens [B], page_tables [B, max_pages]) -> logits."""
        arrs = [np.ascontiguousarray(a, dtype=np.int32) for a in (tokens, positions, page_tables, ctx_lens)]
        _check(lib().decode_step(self.handle, *(_ptr(a) for a in arrs), len(arrs[0]), _ptr(logits),
                                 _stream(stream)))

    def decode_step_device(self, tokens, positions, page_tables, ctx_lens, logits, stream=None) -> None:
        """Same step with int32 device tensors."""
        _check(lib().decode_step_device(self.handle, _ptr(tokens), _ptr(positions), _ptr(page_tables),
                                        _ptr(ctx_lens), tokens.numel(), _ptr(logits), _stream(stream)))

    def w4_device_errors(self, stream=None) -> int:
        return lib().w4_device_errors(self.handle, _stream(stream))

    def w4_model_stage(self, tokens, positions, page_tables, ctx_lens, stream=None) -> None:
        arrs = [None if a is None else np.ascontiguousarray(a, dtype=np.int32)
                for a in (tokens, positions, page_tables, ctx_lens)]
        _check(lib().w4_model_stage(self.handle, *(_ptr(a) for a in arrs), len(arrs[1]), _stream(stream)))

    def w4_model_run_op(self, op: int, layer: int, batch: int, logits=None, stream=None) -> None:
        _check(lib().w4_model_run_op(self.handle, op, layer, batch, _ptr(logits), _stream(stream)))

    def w4_model_buffer(self, which: int):
        """(device address, row stride in fp16 elements) of a workspace buffer."""
        stride = c_int32()
        p = lib().w4_model_buffer(self.handle, which, ctypes.byref(stride))
        return p, stride.value

    def decode_layer(self, layer: int, x_in, x_out, positions, page_tables, ctx_lens, stream=None) -> None:
        arrs = [np.ascontiguousarray(a, dtype=np.int32) for a in (positions, page_tables, ctx_lens)]
        _check(lib().decode_layer(self.handle, layer, _ptr(x_in), _ptr(x_out), *(_ptr(a) for a in arrs),
                                  len(arrs[0]), _stream(stream)))

    def w4_generate_greedy(self, pool: "KvPool", seqs, first_tokens, first_positions, n_steps: int,
                           logits, next_tokens, stream=None) -> np.ndarray:
        """n_steps greedy steps; returns the chosen tokens, int32 [n_steps, B].
        logits: device fp16 [B, vocab]; next_tokens: device int32 [B]."""
        arrs = [np.ascontiguousarray(a, dtype=np.int32) for a in (seqs, first_tokens, first_positions)]
        batch = len(arrs[0])
        out = np.zeros((max(n_steps, 0), batch), dtype=np.int32)
        done = c_int32()
        rc = lib().w4_generate_greedy(self.handle, pool.handle, *(_ptr(a) for a in arrs), batch, n_steps,
                                      _ptr(logits), _ptr(next_tokens), _ptr(out), ctypes.byref(done),
                                      _stream(stream))
        if rc != W4_OK:
            err = W4Error(rc, lib().w4_last_error().decode())
            err.steps_done, err.tokens = done.value, out[:done.value]   # steps whose tokens were chosen
            raise err
        return out


# ------------------------------------------------------------------ kernels

def w4_argmax_workspace_bytes(batch: int, vocab: int) -> int:
    return lib().w4_argmax_workspace_bytes(batch, vocab)


def w4_argmax_f16(logits, out, workspace, stream=None) -> None:
    """out[b] = argmax of logits[b] (lowest index among equal maxima); device
    tensors; workspace >= w4_argmax_workspace_bytes(batch, vocab) bytes."""
    batch, vocab = logits.shape
    _check(lib().w4_argmax_f16(_ptr(logits), batch, vocab, _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _ptr(out), _stream(stream)))


def w4_gemv(packed, x, y, n: int, k: int, batch: int = 1, stream=None) -> None:
    _check(lib().w4_gemv(_ptr(packed), _ptr(x), _ptr(y), n, k, batch, _stream(stream)))


def w4_gemv_f16(packed, x, y, n: int, k: int, batch: int = 1, stream=None) -> None:
    _check(lib().w4_gemv_f16(_ptr(packed), _ptr(x), _ptr(y), n, k, batch, _stream(stream)))


def paged_attention_workspace_bytes(batch, n_heads, n_kv_heads, head_dim, max_pages) -> int:
    return lib().paged_attention_workspace_bytes(batch, n_heads, n_kv_heads, head_dim, max_pages)


def paged_attention_decode(q, k_pool, v_pool, page_tables, ctx_lens, n_heads: int, n_kv_heads: int,
                           head_dim: int, num_pages: int, workspace, out, stream=None) -> None:
    batch, max_pages = page_tables.shape
    _check(lib().paged_attention_decode(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(page_tables),
                                        _ptr(ctx_lens), batch, n_heads, n_kv_heads, head_dim, num_pages,
                                        max_pages, _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _ptr(out),
                                        _stream(stream)))


def paged_attention_decode_noalloc(q, k_pool, v_pool, page_tables, ctx_lens, n_heads: int, n_kv_heads: int,
                                   head_dim: int, num_pages: int, out, stream=None) -> None:
    """paged_attention_decode with the library's own per-device scratch (no workspace)."""
    batch, max_pages = page_tables.shape
    _check(lib().paged_attention_decode_noalloc(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(page_tables),
                                                _ptr(ctx_lens), batch, n_heads, n_kv_heads, head_dim,
                                                num_pages, max_pages, _ptr(out), _stream(stream)))


def w4_prefill_workspace_bytes(cfg: w4_config, max_tokens: int, max_pages: int) -> int:
    return lib().w4_prefill_workspace_bytes(ctypes.byref(cfg), max_tokens, max_pages)


def kv_write_pages(cfg: w4_config, kv_cache, num_pages: int, layer: int, page_table, start: int, k, v,
                   stream=None) -> None:
    """k, v: device fp16 [n][Hkv][D] -> layer `layer` of kv_cache at positions start..start+n-1."""
    _check(lib().kv_write_pages(ctypes.byref(cfg), _ptr(kv_cache), num_pages, layer, _ptr(page_table),
                                page_table.numel(), start, k.shape[0], _ptr(k), _ptr(v), _stream(stream)))


def kv_read_pages(cfg: w4_config, kv_cache, num_pages: int, layer: int, page_table, start: int, k, v,
                  stream=None) -> None:
    """Inverse of kv_write_pages: fills k, v (device fp16 [n][Hkv][D])."""
    _check(lib().kv_read_pages(ctypes.byref(cfg), _ptr(kv_cache), num_pages, layer, _ptr(page_table),
                               page_table.numel(), start, k.shape[0], _ptr(k), _ptr(v), _stream(stream)))


def w4_prefill_buffer(cfg: w4_config, n_tokens: int, max_pages: int, which: int):
    """(byte offset, row stride in fp16 elements) of a prefill workspace buffer."""
    stride = c_int32()
    off = lib().w4_prefill_buffer(ctypes.byref(cfg), n_tokens, max_pages, which, ctypes.byref(stride))
    if off < 0:
        raise W4Error(W4_EINVAL, "w4_prefill_buffer: bad arguments")
    return off, stride.value


def w4_gemv_variant(packed, x, y, n: int, k: int, batch: int = 1, int8_activations: bool = True,
                    stream=None) -> None:
    """W4A8 (int8_activations) or same-decomposition W4A16 GEMV, batch 1..16."""
    _check(lib().w4_gemv_variant(_ptr(packed), _ptr(x), _ptr(y), n, k, batch, int(int8_activations),
                                 _stream(stream)))

