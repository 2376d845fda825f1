"""Teacher-forced, operation-by-operation comparison of the GPU decode path
with the oracle: each operation's stored fp16 output is checked against the
oracle stage fed with the GPU's own inputs to that operation, so every
comparison isolates one kernel's arithmetic (fp16 re-rounding of an
intermediate on either side cannot propagate into later checks)."""
import numpy as np
import torch

import w4a16_paged_kv_amd as w4
from oracle import decode as od
from tests.gpu_util import assert_close, to_np16
from workloads.device import to_dev


def buf(dm, which, batch):
    p, stride = dm.model.w4_model_buffer(which)
    off = p - dm.workspace.data_ptr()
    return dm.workspace[off: off + batch * stride * 2].view(torch.float16).view(batch, stride)


def kv_slot(dm, layer, which, page, slot):
    return to_np16(dm.kv_cache[layer, which, page, :, slot])


def staged_layer(dm, w, layer, x_in, lw, kp, vp, tag="", log=print, live=None):
    """Runs layer `layer` op by op from residual x_in [B, H] (fp16) and checks
    every operation of the sequences in `live` (default: all; a sequence whose
    residual is no longer finite cannot be compared). kp/vp: float64 oracle
    pools of this layer (updated in place with the GPU's K/V). Returns the
    GPU's layer output [B, H]."""
    sh, B, m = w.shape, w.batch, dm.model
    live = np.arange(B) if live is None else np.asarray(live)
    if len(live) < B:
        x_in = x_in.copy()
        x_in[np.setdiff1d(np.arange(B), live)] = 0    # oracle inputs of skipped rows: any finite value
    nq = sh.n_heads * sh.head_dim
    X = buf(dm, w4.BUF_X, B)
    X[live, :sh.hidden] = to_dev(x_in[live])
    m.w4_model_stage(None, w.positions, w.page_tables, w.ctx_lens)

    m.w4_model_run_op(w4.OP_QKV, layer, B)
    torch.cuda.synchronize()
    q_gpu = to_np16(buf(dm, w4.BUF_Q, B)[:, :nq]).reshape(B, sh.n_heads, sh.head_dim)
    xn = to_np16(buf(dm, w4.BUF_XN, B)[:, :sh.hidden])
    assert_close(xn[live], od.rmsnorm(x_in, lw.attn_norm, sh.eps)[live], f"{tag} layer {layer}: rmsnorm")
    q_ref, k_ref, v_ref = od.qkv_from_normed(np.where(np.isfinite(xn), xn, 0), lw, w.positions, sh)
    for b in live:
        pos = int(w.positions[b])
        page, slot = int(w.page_tables[b, pos // 16]), pos % 16
        k_gpu, v_gpu = kv_slot(dm, layer, 0, page, slot), kv_slot(dm, layer, 1, page, slot)
        assert_close(q_gpu[b], q_ref[b], f"{tag} layer {layer} seq {b}: q")
        assert_close(k_gpu, k_ref[b], f"{tag} layer {layer} seq {b}: k")
        assert_close(v_gpu, v_ref[b], f"{tag} layer {layer} seq {b}: v")
        kp[page, :, slot] = k_gpu
        vp[page, :, slot] = v_gpu

    m.w4_model_run_op(w4.OP_ATTN, layer, B)
    torch.cuda.synchronize()
    o_gpu = to_np16(buf(dm, w4.BUF_O, B)[:, :nq])
    for b in live:
        o_ref = od.attention_decode(q_gpu[b], kp, vp, w.page_tables[b], int(w.ctx_lens[b]))
        assert_close(o_gpu[b], o_ref.reshape(-1), f"{tag} layer {layer} seq {b}: attention o")

    m.w4_model_run_op(w4.OP_OPROJ, layer, B)
    torch.cuda.synchronize()
    x1 = to_np16(X[:, :sh.hidden])
    fin = lambda a: np.where(np.isfinite(a), a, 0)
    assert_close(x1[live], od.oproj_stage(x_in, fin(o_gpu), lw)[live], f"{tag} layer {layer}: x + W_o o")
    live = np.array([b for b in live if np.all(np.isfinite(x1[b].astype(np.float64)))], dtype=int)

    m.w4_model_run_op(w4.OP_GATE_UP, layer, B)
    torch.cuda.synchronize()
    h = to_np16(buf(dm, w4.BUF_H, B)[:, :sh.ffn])
    xn2 = to_np16(buf(dm, w4.BUF_XN, B)[:, :sh.hidden])
    assert_close(xn2[live], od.rmsnorm(fin(x1), lw.mlp_norm, sh.eps)[live], f"{tag} layer {layer}: rmsnorm 2")
    assert_close(h[live], od.gate_up_from_normed(fin(xn2), lw, sh)[live], f"{tag} layer {layer}: silu(g) u")
    live = np.array([b for b in live if np.all(np.isfinite(h[b].astype(np.float64)))], dtype=int)

    m.w4_model_run_op(w4.OP_DOWN, layer, B)
    torch.cuda.synchronize()
    x2 = to_np16(X[:, :sh.hidden])
    assert_close(x2[live], od.down_stage(fin(x1), fin(h), lw)[live], f"{tag} layer {layer}: x1 + W_d h")
    log(f"{tag} layer {layer}: q k v o x1 h x2 within tolerance ({len(live)} of {B} sequences compared)")
    return x2
