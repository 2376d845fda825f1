"""paged_attention_decode_noalloc: the allocation-free variant of
paged_attention_decode (its split partials and counters in the library's own
per-device scratch array) must give exactly the workspace entry point's
output, call after call, including a smaller second call that finds the
scratch holding the first call's contents."""
import numpy as np
import pytest
import torch

import w4a16_paged_kv_amd as w4
import workloads as wl
from oracle import runs
from tests.gpu_util import assert_close, to_np16
from workloads.device import k_pages_device, to_dev, v_pages_device


def _poison(k, v, pt, ctx):
    used = np.zeros(k.shape[0], bool)
    for b, c in enumerate(ctx):
        n = (int(c) + 15) // 16
        used[pt[b, :n]] = True
        k[pt[b, n - 1], :, int(c) - (n - 1) * 16:] = np.nan
        v[pt[b, n - 1], :, int(c) - (n - 1) * 16:] = np.nan
    k[~used] = np.nan
    v[~used] = np.nan


def _both(w, q, k, v):
    sh = w.shape
    qd, kd, vd = to_dev(q), to_dev(k_pages_device(k)), to_dev(v_pages_device(v))
    ptd = torch.from_numpy(np.ascontiguousarray(w.page_tables, np.int32)).cuda()
    cd = torch.from_numpy(np.ascontiguousarray(w.ctx_lens, np.int32)).cuda()
    args = (qd, kd, vd, ptd, cd, sh.n_heads, sh.n_kv_heads, sh.head_dim, k.shape[0])
    out_na = torch.full((w.batch, sh.n_heads, sh.head_dim), float("nan"), dtype=torch.float16, device="cuda")
    w4.paged_attention_decode_noalloc(*args, out_na)
    ws = torch.empty(w4.paged_attention_workspace_bytes(w.batch, sh.n_heads, sh.n_kv_heads, sh.head_dim,
                                                        w.max_pages), dtype=torch.uint8, device="cuda")
    out_ws = torch.full_like(out_na, float("nan"))
    w4.paged_attention_decode(*args, ws, out_ws)
    torch.cuda.synchronize()
    return to_np16(out_na), to_np16(out_ws)


@pytest.mark.gpu
def test_noalloc_equals_workspace_entry_point_on_two_calls():
    # first call: the 32-sequence stress workload (contexts 128..8192, tails NaN)
    w = wl.attn_stress()
    q = w.attn_q()
    k, v = w.kv(0)
    _poison(k, v, w.page_tables, w.ctx_lens)
    need = w4.paged_attention_workspace_bytes(w.batch, 28, 4, 128, w.max_pages)
    assert need <= w4.lib().paged_attention_noalloc_max_bytes()
    print(f"no-alloc call 1: batch {w.batch}, contexts {w.ctx_lens.min()}..{w.ctx_lens.max()}, "
          f"{need} bytes of scratch", flush=True)
    a, b = _both(w, q, k, v)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    # second call, smaller: three sequences of another shape, checked against the oracle too
    sh = wl.Shape(hidden=448, n_heads=7, n_kv_heads=1, head_dim=64, ffn=1536, vocab=64, n_layers=1)
    w2 = wl.custom("noalloc2", 95, sh, [37, 1, 130])
    q2 = w2.attn_q()
    k2, v2 = w2.kv(0)
    _poison(k2, v2, w2.page_tables, w2.ctx_lens)
    print(f"no-alloc call 2: batch {w2.batch}, contexts {list(w2.ctx_lens)}", flush=True)
    a2, b2 = _both(w2, q2, k2, v2)
    assert np.array_equal(a2.view(np.uint16), b2.view(np.uint16))
    assert_close(a2, runs.attention_batch(w2, q2, k2, v2), "no-alloc attention (call 2)")


def test_noalloc_refuses_a_call_beyond_its_scratch():
    """Sizes past the per-device array fail with W4_EINVAL before any device
    work (checked on the host, so this runs without a GPU)."""
    lib = w4.lib()
    cap = lib.paged_attention_noalloc_max_bytes()
    assert cap == 16 << 20
    batch, max_pages = 256, 4096
    assert w4.paged_attention_workspace_bytes(batch, 28, 4, 128, max_pages) > cap
    rc = lib.paged_attention_decode_noalloc(None, None, None, None, None, batch, 28, 4, 128, 100000, max_pages,
                                            None, None)
    assert rc == w4.W4_EINVAL
    assert b"more than" in lib.w4_last_error()
