"""The two full 28-layer workloads at their benchmark sizes: batch 1 with a
2048-token context, and batch 16 with contexts uniform over [1024, 4096].

The oracle checks the launch configuration the benchmark times, operation by
operation: the embedding gather bit-exactly, every operation of a sample of
layers against its oracle stage (the GPU's inputs fed in), and the final
RMSNorm + fp16 lm_head on a sample of vocabulary rows. Layers between the
sampled ones run on the GPU only. The full step through decode_step must
reproduce the op-by-op result bit for bit (same kernels, same order)."""
import numpy as np
import pytest
import torch

import w4a16_paged_kv_amd as w4
import workloads as wl
from oracle import decode as od
from oracle import runs
from tests.gpu_util import assert_close, to_np16
from tests.staged import buf, staged_layer
from workloads.device import DeviceModel

pytestmark = pytest.mark.gpu


def full_check(w, check_layers, n_rows=4096):
    sh, B = w.shape, w.batch
    dm = DeviceModel(w, progress=lambda l: print(f"  uploaded layer {l}", flush=True) if l % 7 == 6 else None)
    cache0 = dm.kv_cache.clone()
    m = dm.model
    tokens, pos, pt, ctx = dm.step_inputs()
    m.w4_model_stage(tokens, pos, pt, ctx)
    m.w4_model_run_op(w4.OP_EMBED, 0, B)
    torch.cuda.synchronize()
    X = buf(dm, w4.BUF_X, B)
    x = to_np16(X[:, :sh.hidden])
    assert np.array_equal(x.view(np.uint16), wl.embedding_rows(w.workload_id, sh, tokens).view(np.uint16))
    live = np.arange(B)
    for l in range(sh.n_layers):
        if l in check_layers:
            kp, vp = (a.astype(np.float64) for a in w.kv(l))
            x = staged_layer(dm, w, l, x, w.layer(l), kp, vp, w.name, live=live)
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
                kp, vp = (a.astype(np.float64) for a in w.kv(l))
                x = staged_layer(dm, w, l, x_prev, w.layer(l), kp, vp, w.name + " (overflow)", live=live)
                live = np.array([b for b in live if np.all(np.isfinite(x[b].astype(np.float64)))])
                print(f"  layer {l}: sequences {gone} overflow fp16 on both sides; {len(live)} still compared")
    assert len(live) > 0
    logits = torch.empty((B, sh.vocab), dtype=torch.float16, device="cuda")
    m.w4_model_run_op(w4.OP_LM_HEAD, 0, B, logits)
    torch.cuda.synchronize()
    xf = to_np16(buf(dm, w4.BUF_XN, B)[:, :sh.hidden])
    for b in live:
        assert_close(xf[b], od.rmsnorm(x[b], w.final_norm(), sh.eps), f"{w.name} seq {b}: final rmsnorm")
    rows = np.sort(np.random.default_rng(7).choice(sh.vocab, n_rows, replace=False))
    ref = runs.lm_head_rows(w, xf[live].astype(np.float64), rows)
    got = to_np16(logits)
    assert_close(got[live][:, rows], ref, f"{w.name} logits (rows sampled)")
    print(f"{w.name}: embedding, layers {sorted(check_layers)} op by op, final norm and "
          f"{n_rows} lm_head rows within tolerance", flush=True)

    # decode_step (graph) replays the same kernels: bit-identical logits
    dm.kv_cache.copy_(cache0)
    step_logits = torch.empty_like(logits)
    m.decode_step(tokens, pos, pt, ctx, step_logits)
    torch.cuda.synchronize()
    assert torch.equal(step_logits.view(torch.int16)[live], logits.view(torch.int16)[live])
    assert m.w4_device_errors() == 0


def test_step_b1_full_size():
    full_check(wl.step_b1(), check_layers={0, 13, 27})


def test_step_b16_full_size():
    full_check(wl.step_b16(), check_layers={0, 27}, n_rows=1024)
