"""Teacher-forced, operation-by-operation comparison of the GPU decode path
with the oracle: each operation's stored fp16 output is checked against the
oracle stage fed with the GPU's own inputs to that operation, so every
comparison isolates one kernel's arithmetic (fp16 re-rounding of an
intermediate on either side cannot propagate into later checks)."""
import numpy as np
import torch

import w4a16_paged_kv_amd as w4
import workloads as wl
from oracle import decode as od
from oracle import runs
from tests.gpu_util import assert_close, to_np16
from workloads.device import DeviceModel, k_pages_host, to_dev, v_pages_host


def buf(dm, which, batch):
    p, stride = dm.model.w4_model_buffer(which)
    off = p - dm.workspace.data_ptr()
    return dm.workspace[off: off + batch * stride * 2].view(torch.float16).view(batch, stride)


def kv_slot(dm, layer, which, page, slot):
    """The [Hkv][D] values of one token slot (K and V slices in the device orders)."""
    pool = dm.kv_cache[layer, which]
    host = v_pages_host if which == 1 else k_pages_host
    return to_np16(host(pool[page])[:, slot])


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


def disagreement(a, ref):
    """(share of elements outside |a - ref| <= 2e-3 + 1e-2 |ref|, largest
    |a - ref| over the elements finite on both sides). An element non-finite
    on one side only counts as outside; non-finite on both (the same
    infinity, or NaN on both) counts as agreeing: the synthetic weights can
    overflow fp16, and where they do both sides overflow."""
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    fa, fr = np.isfinite(a), np.isfinite(ref)
    both = fa & fr
    with np.errstate(invalid="ignore"):
        same_nonfinite = ~fa & ~fr & ((np.isnan(a) & np.isnan(ref)) | (a == ref))
        err = np.where(both, np.abs(a - ref), 0.0)
        bad = np.where(both, err > 2e-3 + 1e-2 * np.abs(np.where(both, ref, 0.0)), ~same_nonfinite)
    return float(bad.mean()), float(err.max()) if err.size else 0.0


def check_envelope(gpu, ref, mirror, what, log=print):
    """End to end the GPU's outputs are held to the envelope of two faithful
    fp16 placements: GPU vs oracle must disagree no more (share outside the
    tolerance, largest error) than the oracle's mirror placement (g, u and
    pre-RoPE q/k also rounded) disagrees with the oracle."""
    sg, eg = disagreement(gpu, ref)
    sm, em = disagreement(mirror, ref)
    fin = np.isfinite(np.asarray(ref, dtype=np.float64))
    rms = np.sqrt(np.mean(np.square(np.asarray(ref, dtype=np.float64)[fin]))) if fin.any() else float("nan")
    log(f"{what} end to end: GPU vs oracle {100 * sg:.3f}% outside tolerance, max err {eg:.4g}; "
        f"mirror vs oracle {100 * sm:.3f}%, max err {em:.4g} (rms {rms:.4g}, {np.size(ref)} values, "
        f"{int((~fin).sum())} non-finite in the oracle)", flush=True)
    # every value inside the tolerance meets the contract outright; otherwise
    # the GPU may disagree no more than the mirror placement does
    assert sg == 0.0 or (sg <= sm and eg <= em), \
        f"{what}: GPU disagreement ({sg:.4%}, {eg:.4g}) outside the envelope ({sm:.4%}, {em:.4g})"
    return sg, eg, sm, em


def full_check(w, check_layers, n_rows=None, force_layers=(), chains=False, log=print):
    """A whole decode step op by op: the embedding gather bit-exactly, every
    operation of the layers in check_layers against its oracle stage (the
    GPU's inputs fed in), the final RMSNorm and n_rows lm_head rows (None:
    all); then decode_step (graph) must reproduce the op-by-op logits bit for
    bit.

    force_layers: at these check layers, and before the lm_head if any are
    given, a sequence whose residual is no longer finite (the synthetic
    weights overflow fp16 for some sequences) gets a finite stand-in row
    (workloads.forced_rows), so the layer and its attention over the
    sequence's real context are still compared for every sequence.

    chains: also run the oracle's own chain from the embedding to the logits,
    in the canonical and the mirror placement, and hold decode_step's logits
    for every sequence whose chain stays finite to the envelope of the two
    (check_envelope)."""
    sh, B = w.shape, w.batch
    dm = DeviceModel(w, progress=lambda l: log(f"  uploaded layer {l}", flush=True) if l % 7 == 6 else None)
    cache0 = dm.kv_cache.clone()
    m = dm.model
    tokens, pos, pt, ctx = dm.step_inputs()
    m.w4_model_stage(tokens, pos, pt, ctx)
    m.w4_model_run_op(w4.OP_EMBED, 0, B)
    torch.cuda.synchronize()
    X = buf(dm, w4.BUF_X, B)
    x = to_np16(X[:, :sh.hidden])
    x0 = wl.embedding_rows(w.workload_id, sh, tokens)
    assert np.array_equal(x.view(np.uint16), x0.view(np.uint16))
    live = np.arange(B)
    natural = np.ones(B, bool)       # never fed a stand-in row
    chain = {mir: x0.astype(np.float64) for mir in (False, True)} if chains else {}

    def force(x, layer):
        bad = [b for b in range(B) if not np.all(np.isfinite(x[b].astype(np.float64)))]
        if bad:
            x = x.copy()
            x[bad] = wl.forced_rows(w.workload_id, layer, bad, sh.hidden)
            natural[bad] = False
            X[bad, :sh.hidden] = to_dev(x[bad])
            log(f"  layer {layer}: sequences {bad} overflowed; fed stand-in rows", flush=True)
        return x, np.arange(B)

    for l in range(sh.n_layers):
        lw = w.layer(l)
        kv = w.kv(l)
        for mir in chain:
            chain[mir], _, _ = runs.layer_batch(w, l, chain[mir], pools=tuple(a.astype(np.float64) for a in kv),
                                                weights=lw, mirror=mir)
        if l in check_layers:
            if l in force_layers:
                x, live = force(x, l)
            kp, vp = (a.astype(np.float64) for a in kv)
            x = staged_layer(dm, w, l, x, lw, kp, vp, w.name, live=live, log=log)
            live = np.array([b for b in live if np.all(np.isfinite(x[b].astype(np.float64)))], dtype=int)
        else:
            x_prev = x
            for op in (w4.OP_QKV, w4.OP_ATTN, w4.OP_OPROJ, w4.OP_GATE_UP, w4.OP_DOWN):
                m.w4_model_run_op(op, l, B)
            torch.cuda.synchronize()
            x = to_np16(X[:, :sh.hidden])
            gone = [b for b in live if not np.all(np.isfinite(x[b].astype(np.float64)))]
            if gone:
                # the random-init stack overflowed fp16 for these sequences: check
                # the overflowing layer op by op against the oracle (which must
                # overflow at the same elements), then stop comparing them
                kp, vp = (a.astype(np.float64) for a in kv)
                x = staged_layer(dm, w, l, x_prev, lw, kp, vp, w.name + " (overflow)", live=live, log=log)
                live = np.array([b for b in live if np.all(np.isfinite(x[b].astype(np.float64)))], dtype=int)
                log(f"  layer {l}: sequences {gone} overflow fp16 on both sides; {len(live)} still compared")
    if force_layers:
        x, live = force(x, sh.n_layers)
    assert len(live) > 0
    logits = torch.empty((B, sh.vocab), dtype=torch.float16, device="cuda")
    m.w4_model_run_op(w4.OP_LM_HEAD, 0, B, logits)
    torch.cuda.synchronize()
    xf = to_np16(buf(dm, w4.BUF_XN, B)[:, :sh.hidden])
    if B > 1:
        # the model's lm_head reads the final RMSNorm's rows in the MFMA
        # operand order; the public call reads the same rows as rows: same
        # kernel, same accumulation order, so the same bits
        xrows = buf(dm, w4.BUF_XN, B)[:, :sh.hidden].contiguous()
        again = torch.empty_like(logits)
        w4.w4_gemv_f16(dm.lm_head, xrows, again, sh.vocab, sh.hidden, B)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int16), logits.view(torch.int16)), "lm_head row orders differ"
    for b in live:
        assert_close(xf[b], od.rmsnorm(x[b], w.final_norm(), sh.eps), f"{w.name} seq {b}: final rmsnorm")
    rows = (np.arange(sh.vocab) if n_rows is None else
            np.sort(np.random.default_rng(7).choice(sh.vocab, n_rows, replace=False)))
    # one pass over the regenerated lm_head serves the op-by-op rows and both chains
    xfs = [xf[live].astype(np.float64)]
    for mir in chain:
        xfs.append(np.stack([od.rmsnorm(chain[mir][b], w.final_norm(), sh.eps) for b in range(B)]))
    with np.errstate(invalid="ignore", over="ignore"):
        allref = runs.lm_head_rows(w, np.concatenate(xfs), rows)
    ref = allref[:len(live)]
    got = to_np16(logits)
    assert_close(got[live][:, rows], ref, f"{w.name} logits ({len(rows)} rows)")
    log(f"{w.name}: embedding, layers {sorted(check_layers)} op by op, final norm and "
        f"{len(rows)} lm_head rows within tolerance ({len(live)} of {B} sequences)", flush=True)

    # decode_step (graph) replays the same kernels: bit-identical logits
    dm.kv_cache.copy_(cache0)
    step_logits = torch.empty_like(logits)
    m.decode_step(tokens, pos, pt, ctx, step_logits)
    torch.cuda.synchronize()
    same = [b for b in live if natural[b]]
    assert torch.equal(step_logits.view(torch.int16)[same], logits.view(torch.int16)[same])
    assert m.w4_device_errors() == 0
    if not chain:
        return None
    canon = allref[len(live):len(live) + B]
    mirror = allref[len(live) + B:]
    ok = [b for b in range(B) if natural[b] and np.all(np.isfinite(canon[b])) and np.all(np.isfinite(mirror[b]))]
    assert ok, "no sequence stays finite through the oracle's chain"
    gpu = to_np16(step_logits)[ok][:, :].astype(np.float64)
    return check_envelope(gpu, canon[ok], mirror[ok], f"{w.name} logits of sequences {ok}", log=log)
