"""Benchmark of the W4A16 paged-KV decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload step_b1]

Default workload: the full 28-layer Qwen2.5-7B-shape decode step (random-init
W4A16 weights, fp16 lm_head), batch 1, 2048-token context. One step = one
decode_step over all layers + lm_head for the batch, inputs already resident
in HBM. Prints one JSON line: ms/token, tokens/s, effective HBM GB/s against
the 8 TB/s peak, the roofline of the dominant kernel and the CPU oracle
timed on a bounded sample of the same workload. More workloads are timed and
reported under their own keys: on the same weights the batch-16 step
(step_b16: 16 sequences, contexts 1024..4096) and the prefill of a
512-token prompt (prefill_512: time to first token), and paged attention
alone on 32 sequences with contexts 128..8192 (attn_stress).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12          # MI355X HBM3E, bytes/s
PEAK_MFMA_F16 = 2.5e15     # MI355X dense fp16 matrix peak, flop/s
GEN_STEPS = 16            # greedy generation steps timed after the step itself
ARGMAX_CALLS = 20         # greedy-choice calls per timed graph replay
COPY_BYTES = 1 << 30      # plain copy timed for the measured streaming rate
METRIC = "decode ms/token + effective HBM GB/s (% of peak), Qwen2.5-7B-shape W4A16"


# ------------------------------------------------------------------ byte model

def w4_bytes(n, k):
    return n * k // 2 + n * ((k + 127) // 128) * 2


def op_bytes(sh, batch, ctx_lens):
    """Algorithmic HBM bytes of each operation type for one step (all layers):
    weights read once, activations, KV read and written."""
    H, F, D, Hq, Hkv, V = sh.hidden, sh.ffn, sh.head_dim, sh.n_heads, sh.n_kv_heads, sh.vocab
    L, B = sh.n_layers, batch
    qkv_n = (Hq + 2 * Hkv) * D
    kv_tok = 2 * Hkv * D * 2                     # K and V bytes of one token, one layer
    per = {
        "embed": B * H * 2 * 2,
        "qkv": L * (w4_bytes(qkv_n, H) + H * 2 + B * (H * 2 + Hq * D * 2 + kv_tok)),
        "attn": L * (int(np.sum(ctx_lens)) * kv_tok + B * 2 * Hq * D * 2),
        "oproj": L * (w4_bytes(H, Hq * D) + B * (Hq * D * 2 + 2 * H * 2)),
        "gate_up": L * (w4_bytes(2 * F, H) + H * 2 + B * (H * 2 + F * 2)),
        "down": L * (w4_bytes(H, F) + B * (F * 2 + 2 * H * 2)),
        "lm_head": V * H * 2 + H * 2 + B * (H * 2 + V * 2),
    }
    return per


def prefill_flops(sh, n):
    """Multiply-add work of a prefill of n tokens from position 0 (2 flops per
    multiply-add): every projection for every row, causal attention (scores
    and P V over 1 + 2 + ... + n positions per head), the last row's lm_head."""
    H, F, D, Hq, Hkv = sh.hidden, sh.ffn, sh.head_dim, sh.n_heads, sh.n_kv_heads
    per_row = (Hq + 2 * Hkv) * D * H + H * Hq * D + 2 * F * H + H * F
    attn = 2 * Hq * D * (n * (n + 1) // 2)
    return 2 * sh.n_layers * (n * per_row + attn) + 2 * sh.vocab * H


def attach(dm, w):
    """A second model on dm's uploaded weights, with workload w's KV pages,
    page tables and its own workspace (timing only: the weights' values are
    random draws either way)."""
    import torch
    import w4a16_paged_kv_amd as w4
    from workloads.device import upload_kv
    sh = w.shape
    kv = torch.empty((sh.n_layers, 2, w.num_pages, sh.n_kv_heads, 16, sh.head_dim), dtype=torch.float16,
                     device="cuda")
    for l in range(sh.n_layers):
        upload_kv(w, kv, l)
    ws = torch.empty(w4.w4_workspace_bytes(dm.cfg, w.batch, w.max_pages), dtype=torch.uint8, device="cuda")
    m = w4.Model(dm.cfg, dm.layers, kv, w.num_pages, ws, w.batch, w.max_pages, dm.embed, dm.final_norm,
                 dm.lm_head)
    return m, kv, ws


def launches_per_step(name, sh):
    return 1 if name in ("embed", "lm_head") else sh.n_layers


# ------------------------------------------------------------------ helpers

def source_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "w4a16_paged_kv_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel, digest):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_counters.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_digest") != digest:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, budget_s=30.0):
    """The oracle as it stands, on host cores: whole decoder layers of the same
    workload (weights already generated) and then lm_head row chunks, each
    part scaled to the full step if the time budget stops it early."""
    from threadpoolctl import threadpool_info
    from oracle import decode as od
    from oracle import runs
    import workloads as wl
    sh = w.shape
    x = wl.embedding_rows(w.workload_id, sh, w.tokens()).astype(np.float64)
    layer_s = []
    t_all = time.perf_counter()
    l = 0
    while l < sh.n_layers and (not layer_s or time.perf_counter() - t_all < budget_s * 0.7):
        lw = w.layer(l)
        kp, vp = (a.astype(np.float64) for a in w.kv(l))
        t0 = time.perf_counter()
        x, _, _ = runs.layer_batch(w, l, x, pools=(kp, vp), weights=lw)
        layer_s.append(time.perf_counter() - t0)
        l += 1
    gamma = w.final_norm()
    rows, lm_t, c = 0, 0.0, 0
    while rows < sh.vocab and (rows == 0 or time.perf_counter() - t_all < budget_s):
        blk = wl.lm_head_chunk(w.workload_id, sh, c)
        t0 = time.perf_counter()
        for b in range(w.batch):
            od.lm_head(x[b], gamma, blk, sh.eps)
        lm_t += time.perf_counter() - t0
        rows += blk.shape[0]
        c += 1
    lm_s = lm_t * sh.vocab / rows
    step_s = float(np.mean(layer_s)) * sh.n_layers + lm_s
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": round(step_s * 1e3 / w.batch, 1), "unit": "ms/token", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{len(layer_s)} of {sh.n_layers} decoder layers (float64 oracle, batch {w.batch}, "
                      f"ctx {int(w.ctx_lens.max())}) + {rows} of {sh.vocab} lm_head rows, scaled to one "
                      f"step; {sum(layer_s) + lm_t:.1f} s of CPU work"}


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="step_b1", choices=["step_b1", "step_b16"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the batch-16 step, the prefill, the W4A8 variant and the attention stress workload")
    ap.add_argument("--op-reps", type=int, default=20)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first run three plain device copies of MIB MiB each, so that HBM byte "
                         "counters taken over this run can be scaled by a copy of known size")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the decode step is built "
              "and measured for a single GPU; sharding across GPUs is not part of this library", file=sys.stderr)
        sys.exit(2)

    import torch
    import w4a16_paged_kv_amd as w4
    import workloads as wl
    from workloads.device import DeviceModel

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.empty(n // 2, dtype=torch.float16, device="cuda").fill_(1)   # writes n bytes
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)                                              # reads n, writes n
        torch.cuda.synchronize()
        print(f"[bench] calibration: fill of {n} bytes, then 3 negating copies of {n} bytes",
              file=sys.stderr, flush=True)
        del src, dst

    w = wl.WORKLOADS[args.workload]()
    sh, B = w.shape, w.batch
    t0 = time.time()
    print(f"[bench] building {w.name} on the GPU ...", file=sys.stderr, flush=True)
    dm = DeviceModel(w, progress=lambda l: print(f"[bench]   layer {l} uploaded", file=sys.stderr, flush=True)
                     if l % 7 == 6 else None)
    print(f"[bench] built in {time.time() - t0:.0f} s", file=sys.stderr, flush=True)
    m = dm.model
    tokens, pos, pt, ctx = dm.step_inputs()
    dev = [torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda() for a in (tokens, pos, pt, ctx)]
    logits = torch.empty((B, sh.vocab), dtype=torch.float16, device="cuda")
    stream = torch.cuda.current_stream()

    def timed(fn, iters):
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(iters):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / iters          # ms

    # ---- the step: hipGraph replay, device-resident inputs
    m.w4_set_graph(True)
    step = lambda: m.decode_step_device(*dev, logits)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ms = timed(step, args.steps)
    wall = time.perf_counter() - t_wall
    assert m.w4_device_errors() == 0
    # per-step distribution (one event pair per step, after the timed region)
    per_step = []
    for _ in range(max(20, args.steps // 4)):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        torch.cuda.synchronize()
        per_step.append(a.elapsed_time(b))
    pct = np.percentile(per_step, [10, 50, 90])
    # host-array inputs (includes the staging copies) and eager launches, for context
    host_ms = timed(lambda: m.decode_step(tokens, pos, pt, ctx, logits), max(10, args.steps // 4))
    m.w4_set_graph(False)
    eager_ms = timed(lambda: m.decode_step_device(*dev, logits), max(10, args.steps // 4))
    m.w4_set_graph(True)

    per = op_bytes(sh, B, ctx)
    step_bytes = sum(per.values())

    # ---- per-operation timing: each op type's launches of one step, captured
    # in a graph and replayed (same kernels and arguments as inside the step)
    m.w4_model_stage(tokens, pos, pt, ctx)
    ops = {"embed": (w4.OP_EMBED, [0]), "qkv": (w4.OP_QKV, range(sh.n_layers)),
           "attn": (w4.OP_ATTN, range(sh.n_layers)), "oproj": (w4.OP_OPROJ, range(sh.n_layers)),
           "gate_up": (w4.OP_GATE_UP, range(sh.n_layers)), "down": (w4.OP_DOWN, range(sh.n_layers)),
           "lm_head": (w4.OP_LM_HEAD, [0])}
    op_ms = {}
    for name, (op, layers) in ops.items():
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for l in layers:
                m.w4_model_run_op(op, l, B, logits)
        g.replay()
        op_ms[name] = timed(g.replay, args.op_reps) / len(layers)     # per launch
        del g
    shares = {n: op_ms[n] * launches_per_step(n, sh) for n in op_ms}
    dom = max(shares, key=shares.get)
    dom_bytes = per[dom] / launches_per_step(dom, sh)
    # the sources each operation's kernel is built from (the digest ties the
    # committed counter summary to them)
    gemv_src = ("gemv.hip", "gemv_b1.h", "w4_internal.h")
    kernels = {"qkv": gemv_src, "oproj": gemv_src, "gate_up": gemv_src, "down": gemv_src, "lm_head": gemv_src,
               "embed": gemv_src, "attn": ("attention.hip", "attn_item.h", "gemv_b1.h", "w4_internal.h")}
    digest = source_digest(*kernels[dom])
    achieved = dom_bytes / (op_ms[dom] * 1e-3)

    # ---- greedy generation loop (w4_generate_greedy): the last GEN_STEPS
    # positions of every sequence's context, with pool growth, page tables,
    # the step, the device argmax and one host synchronisation per step; the
    # pool hands out its own pages (every KV slot is an N(0,1) draw, so any
    # page assignment is an equally valid input). Timed by the host clock.
    gen_steps = int(min(GEN_STEPS, ctx.min()))
    nxt = torch.empty((B,), dtype=torch.int32, device="cuda")
    p0 = (ctx - gen_steps).astype(np.int32)

    def generation(n):
        pool = w4.KvPool(w.num_pages, B)
        for b in range(B):
            pool.kv_seq_reserve(b, int(p0[b]))
        torch.cuda.synchronize()
        t = time.perf_counter()
        stop = None
        try:
            toks = m.w4_generate_greedy(pool, list(range(B)), tokens, p0, n, logits, nxt)
            steps = n
        except w4.W4Error as e:
            # the seeded random-init model can overflow the fp16 residual on
            # some trajectories (all logits NaN): that step still ran
            if "NaN" not in str(e):
                raise
            toks, steps, stop = e.tokens, e.steps_done + 1, str(e)
        torch.cuda.synchronize()
        t = time.perf_counter() - t
        pool.close()
        return t, toks, steps, stop

    generation(2)
    gen_s, gen_toks, gen_run, gen_stop = generation(gen_steps)
    assert ((gen_toks >= 0) & (gen_toks < sh.vocab)).all()
    g = torch.cuda.CUDAGraph()
    amax_ws = torch.empty((w4.w4_argmax_workspace_bytes(B, sh.vocab),), dtype=torch.uint8, device="cuda")
    with torch.cuda.graph(g):                     # 20 calls per replay: one replay's own
        for _ in range(ARGMAX_CALLS):             # launch cost is not the kernels' time
            w4.w4_argmax_f16(logits, nxt, amax_ws)
    g.replay()
    argmax_ms = timed(g.replay, args.op_reps) / ARGMAX_CALLS
    del g
    gen = {"steps": gen_run, "ms_per_step": round(gen_s * 1e3 / gen_run, 4),
           "ms_per_token": round(gen_s * 1e3 / gen_run / B, 4), "clock": "host, one sync per step",
           "stopped": gen_stop,
           "argmax_us_per_call": round(argmax_ms * 1e3, 2), "argmax_kernels_per_call": 2,
           "argmax_GBps": round(B * sh.vocab * 2 / (argmax_ms * 1e-3) / 1e9, 1),
           "argmax_bytes_per_call": B * sh.vocab * 2}

    # ---- measured streaming rate of this GPU: a plain device-to-device copy
    # of 1 GiB (reads 1 GiB, writes 1 GiB), for the step's share of what a
    # simple streaming kernel reaches on the same box
    src = torch.empty((COPY_BYTES // 2,), dtype=torch.float16, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    copy_ms = timed(lambda: dst.copy_(src), 10)
    copy_GBps = 2 * COPY_BYTES / (copy_ms * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()

    # ---- batch-16 step on the same weights (graph replay, device inputs)
    b16 = None
    if args.workload == "step_b1" and not args.no_extra:
        w16 = wl.step_b16()
        m16, kv16, ws16 = attach(dm, w16)
        t16, p16, pt16, c16 = w16.tokens(), w16.positions, w16.page_tables, w16.ctx_lens
        dev16 = [torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda() for a in (t16, p16, pt16, c16)]
        lg16 = torch.empty((w16.batch, sh.vocab), dtype=torch.float16, device="cuda")
        s16 = lambda: m16.decode_step_device(*dev16, lg16)
        for _ in range(5):
            s16()
        ms16 = timed(s16, max(10, args.steps // 4))
        bytes16 = sum(op_bytes(sh, w16.batch, c16).values())
        b16 = {"ms_per_step": round(ms16, 4), "ms_per_token": round(ms16 / w16.batch, 4),
               "tokens_per_s": round(w16.batch * 1e3 / ms16, 1), "bytes_per_step": int(bytes16),
               "effective_GBps": round(bytes16 / (ms16 * 1e-3) / 1e9, 1),
               "pct_of_peak": round(100 * bytes16 / (ms16 * 1e-3) / PEAK_HBM, 2),
               "ctx": {"min": int(c16.min()), "max": int(c16.max()), "sum": int(c16.sum())},
               "graph": True, "inputs": "device"}
        m16.close()
        del kv16, ws16, dev16, lg16
        print(f"[bench] step_b16 {ms16:.4f} ms/step", file=sys.stderr, flush=True)

    # ---- prefill of a 512-token prompt (time to first token), same weights
    pf = None
    if args.workload == "step_b1" and not args.no_extra:
        wp = wl.prefill_512()
        mp, kvp, wsp = attach(dm, wp)
        n = int(wp.ctx_lens[0])
        ptok = wp.prompt_tokens(n)
        pws = torch.empty(w4.w4_prefill_workspace_bytes(dm.cfg, n, wp.max_pages), dtype=torch.uint8, device="cuda")
        plog = torch.empty(sh.vocab, dtype=torch.float16, device="cuda")
        run_pf = lambda: mp.w4_prefill(ptok, 0, wp.page_tables[0], pws, plog)
        for _ in range(2):
            run_pf()
        torch.cuda.synchronize()
        reps = 10
        t = time.perf_counter()
        for _ in range(reps):
            run_pf()
        torch.cuda.synchronize()
        ttft = (time.perf_counter() - t) / reps * 1e3
        gpu_ms = timed(run_pf, reps)
        fl = prefill_flops(sh, n)
        pf = {"tokens": n, "ttft_ms": round(ttft, 3), "clock": "host, prompt on the host to logits on the device",
              "gpu_ms": round(gpu_ms, 3), "flop": int(fl),
              "TFLOPs": round(fl / (gpu_ms * 1e-3) / 1e12, 1),
              "pct_of_mfma_peak": round(100 * fl / (gpu_ms * 1e-3) / PEAK_MFMA_F16, 2),
              "tokens_per_s": round(n * 1e3 / ttft, 1)}
        mp.close()
        del kvp, wsp, pws, plog
        print(f"[bench] prefill_512 {ttft:.3f} ms", file=sys.stderr, flush=True)

    # ---- the W4A8 variant against the W4A16 arithmetic (same one-wavefront-
    # per-tile decomposition) and the step's own projection kernel, on this
    # layer-0 weights' gate/up and down shapes
    variants = None
    if args.workload == "step_b1" and not args.no_extra:
        variants = {}
        lw0 = w.layer(0)
        for name, (qq, ss), n_, k_ in (("gate_up", (lw0.gate_up_q, lw0.gate_up_s), 2 * sh.ffn, sh.hidden),
                                       ("down", (lw0.down_q, lw0.down_s), sh.hidden, sh.ffn)):
            packed = torch.from_numpy(w4.pack_weights_w4g128(qq, ss)).cuda()
            for bsz in ((1, 16) if name == "gate_up" else (1,)):
                xv = torch.randn((bsz, k_), device="cuda").half()
                yv = torch.empty((bsz, n_), dtype=torch.float16, device="cuda")
                res = {}
                for label, fn in (("w4a8_us", lambda: w4.w4_gemv_variant(packed, xv, yv, n_, k_, bsz, True)),
                                  ("w4a16_same_split_us", lambda: w4.w4_gemv_variant(packed, xv, yv, n_, k_, bsz, False)),
                                  ("w4a16_decode_kernel_us", lambda: w4.w4_gemv(packed, xv, yv, n_, k_, bsz))):
                    fn()                      # first call outside the capture (launch attributes)
                    torch.cuda.synchronize()
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g):
                        for _ in range(10):
                            fn()
                    g.replay()
                    res[label] = round(timed(g.replay, args.op_reps) / 10 * 1e3, 2)
                    del g
                res["bytes"] = int(w4_bytes(n_, k_))
                variants[f"{name}_b{bsz}"] = res
            del packed
        print(f"[bench] variants {variants}", file=sys.stderr, flush=True)

    # ---- paged attention alone on 32 sequences with contexts U[128, 8192]
    # (one layer's KV pool), warm: ten calls captured in a graph and replayed
    stress = None
    if args.workload == "step_b1" and not args.no_extra:
        from workloads.device import to_dev, v_pages_device
        ws_ = wl.attn_stress()
        ssh, nseq = ws_.shape, len(ws_.ctx_lens)
        kq, vq = ws_.kv(0)
        qd, kd, vd = to_dev(ws_.attn_q()), to_dev(kq), to_dev(v_pages_device(vq))
        ptd = torch.from_numpy(np.ascontiguousarray(ws_.page_tables, np.int32)).cuda()
        cd = torch.from_numpy(np.ascontiguousarray(ws_.ctx_lens, np.int32)).cuda()
        aws = torch.empty((w4.paged_attention_workspace_bytes(nseq, ssh.n_heads, ssh.n_kv_heads, ssh.head_dim,
                                                              ws_.page_tables.shape[1]),),
                          dtype=torch.uint8, device="cuda")
        aout = torch.empty((nseq, ssh.n_heads, ssh.head_dim), dtype=torch.float16, device="cuda")
        call = lambda: w4.paged_attention_decode(qd, kd, vd, ptd, cd, ssh.n_heads, ssh.n_kv_heads,
                                                 ssh.head_dim, kq.shape[0], aws, aout)
        call()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(10):
                call()
        g.replay()
        reps = [timed(g.replay, 1) / 10 for _ in range(max(10, args.op_reps))]
        us = float(np.median(reps)) * 1e3
        sbytes = int(ws_.ctx_lens.sum()) * ssh.n_kv_heads * ssh.head_dim * 2 * 2 \
            + nseq * ssh.n_heads * ssh.head_dim * 2 * 2
        stress = {"us_per_call": round(us, 2), "sequences": nseq,
                  "ctx": {"min": int(ws_.ctx_lens.min()), "max": int(ws_.ctx_lens.max()),
                          "sum": int(ws_.ctx_lens.sum())},
                  "bytes_per_call": sbytes, "GBps": round(sbytes / (us * 1e-6) / 1e9, 1),
                  "pct_of_peak": round(100 * sbytes / (us * 1e-6) / PEAK_HBM, 2),
                  "clock": "events around one replay of ten captured calls, median of the replays"}
        del g, qd, kd, vd, ptd, cd, aws, aout
        torch.cuda.empty_cache()
        print(f"[bench] attn_stress {us:.2f} us/call", file=sys.stderr, flush=True)

    cpu = None if args.no_cpu else cpu_baseline(w)

    tok_s = B * 1e3 / ms
    out = {
        "metric": METRIC,
        "value": round(ms / B, 4),
        "unit": "ms/token",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic (seeded random-init weights and KV, no checkpoint)",
        "config": {"workload": w.name, "layers": sh.n_layers, "hidden": sh.hidden, "heads": sh.n_heads,
                   "kv_heads": sh.n_kv_heads, "head_dim": sh.head_dim, "ffn": sh.ffn, "vocab": sh.vocab,
                   "batch": B, "ctx": [int(c) for c in ctx] if B <= 4 else
                   {"min": int(ctx.min()), "max": int(ctx.max()), "sum": int(ctx.sum())},
                   "weights": "int4 g128 symmetric, fp16 lm_head", "graph": True, "inputs": "device"},
        "tokens_per_s": round(tok_s, 1),
        "effective_GBps": round(step_bytes / (ms * 1e-3) / 1e9, 1),
        "pct_of_peak": round(100 * step_bytes / (ms * 1e-3) / PEAK_HBM, 2),
        "bytes_per_step": int(step_bytes),
        "measured_copy_GBps": round(copy_GBps, 1),
        "pct_of_measured_copy": round(100 * step_bytes / (ms * 1e-3) / 1e9 / copy_GBps, 2),
        "ms_per_step_p10_p50_p90": [round(float(v), 4) for v in pct],
        "ms_per_step_host_inputs": round(host_ms, 4),
        "ms_per_step_eager": round(eager_ms, 4),
        "wall_s_timed": round(wall, 3),
        "ops": {n: {"us_per_launch": round(op_ms[n] * 1e3, 2), "launches": launches_per_step(n, sh),
                    "GBps": round(per[n] / launches_per_step(n, sh) / (op_ms[n] * 1e-3) / 1e9, 1),
                    "share_of_step": round(shares[n] / ms, 3)} for n in op_ms},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved / 1e9, 1),
                     "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": round(achieved / PEAK_HBM, 4),
                     "traffic": read_traffic(dom, digest), "bytes_per_launch": int(dom_bytes),
                     "us_per_launch": round(op_ms[dom] * 1e3, 2), "source_digest": digest},
        "generate": gen,
        "step_b16": b16,
        "prefill_512": pf,
        "w4a8_variant": variants,
        "attn_stress": stress,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
