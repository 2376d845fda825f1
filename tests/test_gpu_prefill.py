"""Prefill on the GPU (w4_prefill, the prefill GEMM through w4_gemv, the KV
page copies) against the oracle's prefill ("How to build your own LLM runtime
from scratch", Key performance metrics: time to first token of a 512-token
prompt). The oracle's prefill is pinned equal to token-by-token decode
(tests/test_prefill_oracle.py)."""
import numpy as np
import pytest
import torch

import w4a16_paged_kv_amd as w4
import workloads as wl
from oracle import decode as od
from oracle import prefill as op
from oracle import runs
from tests.gpu_util import assert_close, to_np16
from tests.staged import check_envelope
from workloads.device import DeviceModel, k_pages_device, k_pages_host, to_dev, v_pages_device, v_pages_host

pytestmark = pytest.mark.gpu

SMALL = wl.Shape(hidden=448, n_heads=7, n_kv_heads=1, head_dim=64, ffn=1536, vocab=5000, n_layers=3)


# ------------------------------------------------------------- prefill GEMM

@pytest.mark.parametrize("n,k,m", [(576, 448, 37), (3072, 448, 17), (448, 1536, 130), (40, 200, 300),
                                   (4608, 3584, 512), (3584, 3584, 512), (37888, 3584, 512),
                                   (3584, 18944, 512), (3584, 3584, 129), (40000, 200, 300),
                                   (33000, 1000, 257)])
def test_prefill_gemm_matches_oracle(n, k, m):
    """w4_gemv with more than 16 rows runs the prefill GEMM: 32-row tiles with
    a three-stage ring, or (1024 and more 64-row workgroups: the gate/up shape,
    40000 x 200 and 33000 x 1000) 64-row tiles with a two-stage ring; partial
    row tiles, partial last groups (k = 448, 200, 1000)."""
    print(f"prefill gemm n={n} k={k} rows={m}", flush=True)
    q, s = wl.int4_matrix(81, 0, 0, n, k)
    x = wl.f16_normal(wl.rng(81, 0, 1), (m, k))
    y = torch.full((m, n), float("nan"), dtype=torch.float16, device="cuda")
    w4.w4_gemv(to_dev(w4.pack_weights_w4g128(q, s)), to_dev(x), y, n, k, m)
    torch.cuda.synchronize()
    rows = np.arange(m) if m * n <= 4_000_000 else np.random.default_rng(1).choice(m, 48, replace=False)
    assert_close(to_np16(y)[rows], od.r16(od.gemv_w4(q, s, x[rows])), f"prefill gemm {n}x{k}, {m} rows")


# -------------------------------------------------------------- page copies

def test_kv_pages_write_read_round_trip_and_layout():
    """kv_write_pages puts natural-layout K/V rows at their page slots in the
    cache's layouts (K in score operand order, V in P V operand order) and
    nothing else;
    kv_read_pages gives them back; a token whose page id is invalid is
    skipped."""
    cfg = w4.make_config(448, 7, 2, 64, 1536, 100, 3, 1e-6, 1e6)
    P, hkv, d, layer = 9, 2, 64, 1
    cache = torch.randn((3, 2, P, hkv, 16, d), device="cuda").half()
    before = cache.clone()
    pt_host = np.array([4, 7, 0, 8, -1], np.int32)     # position 64..79 -> invalid page
    pt = torch.from_numpy(pt_host).cuda()
    start, n = 5, 70
    rs = np.random.default_rng(2)
    k = rs.standard_normal((n, hkv, d)).astype(np.float16)
    v = rs.standard_normal((n, hkv, d)).astype(np.float16)
    w4.kv_write_pages(cfg, cache, P, layer, pt, start, to_dev(k), to_dev(v))
    torch.cuda.synchronize()
    expect = before.cpu().numpy().view(np.uint16).copy()
    kc, vc = expect[layer, 0], expect[layer, 1]
    for i in range(n):
        p = start + i
        page = pt_host[p // 16]
        if page < 0:
            continue
        mask = np.zeros((hkv, 16, d), bool)
        mask[:, p % 16] = True
        for dst, row, to_device in ((kc, k[i], k_pages_device), (vc, v[i], v_pages_device)):
            h = np.zeros((hkv, 16, d), np.uint16)
            h[:, p % 16] = row.view(np.uint16)
            hd = to_device(h.view(np.float16)).view(np.uint16)
            md = to_device(mask)
            dst[page][md] = hd[md]
    got = cache.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, expect)
    kb = torch.empty((n, hkv, d), dtype=torch.float16, device="cuda")
    vb = torch.empty_like(kb)
    w4.kv_read_pages(cfg, cache, P, layer, pt, start, kb, vb)
    torch.cuda.synchronize()
    ok = np.array([pt_host[(start + i) // 16] >= 0 for i in range(n)])
    assert np.array_equal(to_np16(kb)[ok].view(np.uint16), k[ok].view(np.uint16))
    assert np.array_equal(to_np16(vb)[ok].view(np.uint16), v[ok].view(np.uint16))


# -------------------------------------------------------------- whole prefill

def prefill(dm, tokens, start, keep_ws=False):
    w = dm.w
    ws = torch.empty(w4.w4_prefill_workspace_bytes(dm.cfg, len(tokens), w.max_pages), dtype=torch.uint8,
                     device="cuda")
    logits = torch.empty(w.shape.vocab, dtype=torch.float16, device="cuda")
    dm.model.w4_prefill(tokens, start, w.page_tables[0], ws, logits)
    torch.cuda.synchronize()
    return (to_np16(logits), ws) if keep_ws else to_np16(logits)


def ws_rows(dm, ws, n, which, width):
    off, stride = w4.w4_prefill_buffer(dm.cfg, n, dm.w.max_pages, which)
    return to_np16(ws[off: off + n * stride * 2].view(torch.float16).view(n, stride)[:, :width])


def check_prefill_attention(dm, ws, tokens, start, tag):
    """Teacher-forced check of the prefill attention kernel: every prompt
    row's output of the last layer against the oracle's attention fed the
    GPU's own queries (after RoPE) and the GPU's pages of that layer."""
    sh, n = dm.w.shape, len(tokens)
    nq = sh.n_heads * sh.head_dim
    q = ws_rows(dm, ws, n, w4.BUF_Q, nq).reshape(n, sh.n_heads, sh.head_dim)
    o = ws_rows(dm, ws, n, w4.BUF_O, nq)
    layer = sh.n_layers - 1
    kp = k_pages_host(to_np16(dm.kv_cache[layer, 0])).astype(np.float64)
    vp = v_pages_host(to_np16(dm.kv_cache[layer, 1])).astype(np.float64)
    pt = dm.w.page_tables[0]
    ref = np.stack([od.attention_decode(q[i], kp, vp, pt, start + i + 1).reshape(-1) for i in range(n)])
    assert_close(o, ref, f"{tag}: prefill attention (teacher-forced)")


def read_rows(dm, layer, start, n):
    """The K/V rows [n, Hkv, D] of positions start.. of sequence 0 from the GPU cache."""
    sh = dm.w.shape
    pt = torch.from_numpy(np.ascontiguousarray(dm.w.page_tables[0], np.int32)).cuda()
    kb = torch.empty((n, sh.n_kv_heads, sh.head_dim), dtype=torch.float16, device="cuda")
    vb = torch.empty_like(kb)
    w4.kv_read_pages(dm.cfg, dm.kv_cache, dm.num_pages, layer, pt, start, kb, vb)
    torch.cuda.synchronize()
    return to_np16(kb), to_np16(vb)


def oracle_rows(pools, pt_row, start, n):
    k = np.stack([od.gather_kv(pools[0], pt_row, start + n, j)[start:] for j in range(pools[0].shape[1])], 1)
    v = np.stack([od.gather_kv(pools[1], pt_row, start + n, j)[start:] for j in range(pools[1].shape[1])], 1)
    return k, v


@pytest.mark.parametrize("start,n", [(0, 1), (0, 37), (5, 60), (16, 130), (3, 16)])
def test_prefill_small_model_matches_oracle(start, n):
    """Logits of the last prompt token and every prompt K/V slot of every
    layer against the oracle's prefill (prior context from the workload's
    pages when start > 0); slots outside the prompt keep their bits."""
    w = wl.custom("prefill_small", 40, SMALL, [start + n], layers=3, lm_head=True, gamma="random")
    dm = DeviceModel(w)
    before = dm.kv_cache.clone()
    tokens = w.prompt_tokens(n)
    got, ws = prefill(dm, tokens, start, keep_ws=True)
    check_prefill_attention(dm, ws, tokens, start, f"start={start} n={n}")
    ref = runs.prefill_run(w, tokens, start, keep_pools=True)
    mir = runs.prefill_run(w, tokens, start, mirror=True, keep_pools=True)
    check_envelope(got, ref["logits"], mir["logits"], f"prefill start={start} n={n} logits")
    check_envelope(ws_rows(dm, ws, n, w4.BUF_X, SMALL.hidden), ref["x"], mir["x"], "final residual rows")
    check_kv(dm, ref, mir, start, n, 3)
    for l in range(3):   # prior context: untouched
        if start:
            kb, vb = read_rows(dm, l, 0, start)
            k0 = np.stack([w.kv(l)[0][w.page_tables[0][t // 16], :, t % 16] for t in range(start)])
            assert np.array_equal(kb.view(np.uint16), k0.view(np.uint16))
    changed = (dm.kv_cache.view(torch.int16) != before.view(torch.int16)).any(dim=-1).any(dim=-1)   # [L,2,P,Hkv]
    touched = {int(w.page_tables[0][p // 16]) for p in range(start, start + n)}
    assert not changed[:, :, [p for p in range(w.num_pages) if p not in touched]].any()


SPLIT = wl.Shape(hidden=448, n_heads=7, n_kv_heads=1, head_dim=64, ffn=8320, vocab=5000, n_layers=2)


def test_prefill_split_down_projection_matches_oracle():
    """The down projection split over four workgroups (65 groups of 128
    columns: 16, 16, 16 and 17 per split, partial sums added in split order by
    the last to arrive) with a partial 64-row block (70 prompt rows) and a
    partial 8-tile block (448 outputs): logits, final residual rows and every
    prompt K/V slot against the oracle's prefill; a second prefill gives
    identical bits (the split order does not depend on arrival order)."""
    w = wl.custom("prefill_split", 43, SPLIT, [3 + 70], layers=2, lm_head=True, gamma="random")
    dm = DeviceModel(w)
    tokens = w.prompt_tokens(70)
    got, ws = prefill(dm, tokens, 3, keep_ws=True)
    x1 = ws_rows(dm, ws, 70, w4.BUF_X, SPLIT.hidden)
    got2, ws2 = prefill(dm, tokens, 3, keep_ws=True)
    assert np.array_equal(got.view(np.uint16), got2.view(np.uint16))
    assert np.array_equal(x1.view(np.uint16), ws_rows(dm, ws2, 70, w4.BUF_X, SPLIT.hidden).view(np.uint16))
    ref = runs.prefill_run(w, tokens, 3, keep_pools=True)
    mir = runs.prefill_run(w, tokens, 3, mirror=True, keep_pools=True)
    check_envelope(got, ref["logits"], mir["logits"], "split prefill logits")
    check_envelope(x1, ref["x"], mir["x"], "split prefill final residual rows")
    check_kv(dm, ref, mir, 3, 70, 2)


def check_kv(dm, ref, mir, start, n, layers):
    """Every prompt K/V slot of every layer: layer 0 element by element (one
    operation from the embedding), deeper layers (the end of a chain of
    layers) within the envelope of the oracle's two placements."""
    pt = dm.w.page_tables[0]
    for l in range(layers):
        k, v = read_rows(dm, l, start, n)
        kr, vr = oracle_rows(ref["pools"][l], pt, start, n)
        if l == 0:
            assert_close(k, kr, "layer 0 K of the prompt")
            assert_close(v, vr, "layer 0 V of the prompt")
        else:
            km, vm = oracle_rows(mir["pools"][l], pt, start, n)
            check_envelope(k, kr, km, f"layer {l} K of the prompt")
            check_envelope(v, vr, vm, f"layer {l} V of the prompt")


def test_prefill_then_decode_step_continues_the_sequence():
    """Prefill of n tokens then one decode_step at position n equals the
    oracle's prefill of n + 1 tokens (pinned equal to token-by-token decode)."""
    n = 45
    w = wl.custom("prefill_dec", 41, SMALL, [n + 1], layers=3, lm_head=True, gamma="random")
    dm = DeviceModel(w)
    tokens = w.prompt_tokens(n + 1)
    prefill(dm, tokens[:n], 0)
    logits = torch.empty((1, SMALL.vocab), dtype=torch.float16, device="cuda")
    dm.model.decode_step(tokens[n:], np.array([n], np.int32), w.page_tables, np.array([n + 1], np.int32), logits)
    torch.cuda.synchronize()
    ref = runs.prefill_run(w, tokens, 0)["logits"]
    mir = runs.prefill_run(w, tokens, 0, mirror=True)["logits"]
    check_envelope(to_np16(logits)[0], ref, mir, "decode after prefill")


FULL1 = wl.Shape(hidden=3584, n_heads=28, n_kv_heads=4, head_dim=128, ffn=18944, vocab=32768, n_layers=1)


@pytest.mark.timeout(900)
def test_prefill_512_full_shape_layer():
    """512-token prompt through one decoder layer at the Qwen2.5-7B shape
    (32768-row lm_head; one layer, because past the first layer the
    synthetic weights overflow fp16 for many prompt rows, on both sides):
    the attention kernel teacher-forced on all 512 rows, every prompt K/V
    slot element by element, and the final residual rows and the last
    token's logits within the envelope of the oracle's two placements."""
    w = wl.custom("prefill_full1", 42, FULL1, [512], layers=1, lm_head=True)
    dm = DeviceModel(w)
    tokens = w.prompt_tokens(512)
    got, ws = prefill(dm, tokens, 0, keep_ws=True)
    print("prefill 512 (full-shape layer) on the GPU done; oracle running", flush=True)
    check_prefill_attention(dm, ws, tokens, 0, "full shape, 512 rows")
    ref = runs.prefill_run(w, tokens, 0, keep_pools=True)
    mir = runs.prefill_run(w, tokens, 0, mirror=True, keep_pools=True)
    check_envelope(got, ref["logits"], mir["logits"], "prefill 512 full shape logits")
    assert np.all(np.isfinite(ref["x"]))
    check_envelope(ws_rows(dm, ws, 512, w4.BUF_X, FULL1.hidden), ref["x"], mir["x"], "final residual rows")
    check_kv(dm, ref, mir, 0, 512, 1)


@pytest.mark.timeout(900)
def test_prefill_512_benchmark_model_first_layer():
    """The benchmark's configuration (28 layers, 152064-row lm_head, 512
    tokens): every prompt K/V slot of layer 0 against the oracle's first
    prefill layer; a second prefill gives identical bits. (Deeper layers run
    the same kernels with the same launch shapes as the one-layer test; past
    the first layer the synthetic weights overflow fp16 for many rows.)"""
    w = wl.prefill_512()
    dm = DeviceModel(w, progress=lambda l: print(f"  uploaded layer {l}", flush=True) if l % 7 == 6 else None)
    tokens = w.prompt_tokens(512)
    got = prefill(dm, tokens, 0)
    kp, vp = runs.pools_f64(w, 0)
    x0 = wl.embedding_rows(w.workload_id, w.shape, tokens)
    op.prefill_layer(x0, w.layer(0), kp, vp, w.page_tables[0], 0, w.shape)
    k, v = read_rows(dm, 0, 0, 512)
    kr, vr = oracle_rows((kp, vp), w.page_tables[0], 0, 512)
    assert_close(k, kr, "prefill_512 layer 0 K")
    assert_close(v, vr, "prefill_512 layer 0 V")
    again = prefill(dm, tokens, 0)
    assert np.array_equal(got.view(np.uint16), again.view(np.uint16))
