"""Paged-attention decode kernel against the oracle, plus the page-indexing
regressions ("Building a Custom LLM Inference Runtime on H100", The Three
Critical Bugs, Bug 1; "How to build your own LLM runtime from scratch",
Architectural decisions: barriers in divergent branches corrupted page tails)."""
import numpy as np
import pytest
import torch

import w4a16_paged_kv_amd as w4
import workloads as wl
from oracle import runs
from tests.gpu_util import assert_close, to_np16
from workloads.device import k_pages_device, to_dev, v_pages_device

pytestmark = pytest.mark.gpu


def run_attn(q, k, v, pt, ctx, n_heads, n_kv, d):
    qd, kd, vd = to_dev(q), to_dev(k_pages_device(k)), to_dev(v_pages_device(v))
    ptd = torch.from_numpy(np.ascontiguousarray(pt, np.int32)).cuda()
    cd = torch.from_numpy(np.ascontiguousarray(ctx, np.int32)).cuda()
    ws = torch.empty(w4.paged_attention_workspace_bytes(len(ctx), n_heads, n_kv, d, pt.shape[1]),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((len(ctx), n_heads, d), dtype=torch.float16, device="cuda")
    w4.paged_attention_decode(qd, kd, vd, ptd, cd, n_heads, n_kv, d, k.shape[0], ws, out)
    torch.cuda.synchronize()
    return to_np16(out)


def poison(k, v, pt, ctx, value=np.nan):
    """Fill every slot no context token occupies (tails of last pages, unused pages)."""
    used = np.zeros(k.shape[0], bool)
    for b, c in enumerate(ctx):
        n = (int(c) + 15) // 16
        ids = pt[b, :n]
        used[ids] = True
        tail = int(c) - (n - 1) * 16
        k[ids[-1], :, tail:] = value
        v[ids[-1], :, tail:] = value
    k[~used] = value
    v[~used] = value


def test_attention_stress_workload():
    """32 sequences, contexts uniform over [128, 8192], tails NaN-poisoned."""
    w = wl.attn_stress()
    sh = w.shape
    q = w.attn_q()
    k, v = w.kv(0)
    poison(k, v, w.page_tables, w.ctx_lens)
    print("attn_stress: contexts", w.ctx_lens.min(), w.ctx_lens.max(), "pages", w.num_pages, flush=True)
    got = run_attn(q, k, v, w.page_tables, w.ctx_lens, sh.n_heads, sh.n_kv_heads, sh.head_dim)
    ref = runs.attention_batch(w, q, k, v)
    assert_close(got, ref, "attn_stress")


@pytest.mark.parametrize("d,hq,hkv", [(128, 28, 4), (64, 7, 1), (128, 8, 8), (64, 16, 2), (128, 16, 4), (64, 8, 1)])
def test_ragged_contexts_all_tails(d, hq, hkv):
    """Context lengths 1..40 and around page boundaries: every tail length."""
    ctx = np.array(list(range(1, 41)) + [63, 64, 65, 127, 128, 129, 255, 256, 257], np.int32)
    sh = wl.Shape(hidden=hq * d, n_heads=hq, n_kv_heads=hkv, head_dim=d, ffn=8, vocab=8, n_layers=1)
    w = wl.custom("ragged", 60 + d + hq, sh, ctx)
    q = w.attn_q()
    k, v = w.kv(0)
    poison(k, v, w.page_tables, w.ctx_lens, np.inf)
    got = run_attn(q, k, v, w.page_tables, w.ctx_lens, hq, hkv, d)
    assert_close(got, runs.attention_batch(w, q, k, v), f"ragged d={d} gqa={hq // hkv}")


@pytest.mark.parametrize("ctx", [300, 4000, 16384])
def test_many_splits_reach_the_merge(ctx):
    """One sequence, one KV head: the context is split into 3, 32 and 128
    splits of 8 pages, so the merging workgroup combines every count of
    partials up to its limit (128), with a partial last page."""
    sh = wl.Shape(hidden=896, n_heads=7, n_kv_heads=1, head_dim=128, ffn=8, vocab=8, n_layers=1)
    w = wl.custom("splits", 66, sh, [ctx - 5])
    q = w.attn_q()
    k, v = w.kv(0)
    poison(k, v, w.page_tables, w.ctx_lens)
    got = run_attn(q, k, v, w.page_tables, w.ctx_lens, 7, 1, 128)
    assert_close(got, runs.attention_batch(w, q, k, v), f"{ctx - 5} tokens")


def test_tail_poison_does_not_change_the_result():
    w = wl.custom("tails", 61, wl.QWEN7B, [17, 31, 200, 333, 1000], 0)
    q = w.attn_q()
    k, v = w.kv(0)
    a = run_attn(q, k, v, w.page_tables, w.ctx_lens, 28, 4, 128)
    poison(k, v, w.page_tables, w.ctx_lens, np.nan)
    b = run_attn(q, k, v, w.page_tables, w.ctx_lens, 28, 4, 128)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_page_permutation_is_bit_identical():
    """The same logical KV placed through two different page tables gives
    bit-identical outputs."""
    sh = wl.QWEN7B
    ctx = np.array([700, 1234, 16, 5], np.int32)
    w = wl.custom("perm", 62, sh, ctx, 0)
    q = w.attn_q()
    k, v = w.kv(0)
    pt2 = w.page_tables.copy()
    perm = np.random.default_rng(5).permutation(w.num_pages)
    k2, v2 = np.empty_like(k), np.empty_like(v)
    k2[perm] = k
    v2[perm] = v
    live = pt2 >= 0
    pt2[live] = perm[pt2[live]]
    a = run_attn(q, k, v, w.page_tables, ctx, 28, 4, 128)
    b = run_attn(q, k2, v2, pt2, ctx, 28, 4, 128)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


@pytest.mark.parametrize("tstar", [0, 14, 15, 16, 17, 31, 32, 33, 95, 99])
def test_argmax_probe_reads_exactly_the_probed_slot(tstar):
    """One token with a dominant score: o equals its V row (fp16-exact)."""
    d, ctx = 128, 100
    sh = wl.Shape(hidden=7 * d, n_heads=7, n_kv_heads=1, head_dim=d, ffn=8, vocab=8, n_layers=1)
    w = wl.custom("probe", 63, sh, [ctx])
    k, v = w.kv(0)
    k[:] = 0
    page, slot = w.page_tables[0, tstar // 16], tstar % 16
    k[page, 0, slot, 0] = 64.0
    q = np.zeros((1, 7, d), np.float16)
    q[0, :, 0] = 64.0          # score gap 64*64/sqrt(128) = 362 -> other weights underflow
    got = run_attn(q, k, v, w.page_tables, w.ctx_lens, 7, 1, d)
    assert np.array_equal(got[0], np.repeat(v[page, 0, slot][None], 7, axis=0))


def test_closed_forms_ctx1_and_constant_v():
    sh = wl.Shape(hidden=28 * 128, n_heads=28, n_kv_heads=4, head_dim=128, ffn=8, vocab=8, n_layers=1)
    w = wl.custom("closed", 64, sh, [1, 50])
    q = w.attn_q()
    k, v = w.kv(0)
    got = run_attn(q, k, v, w.page_tables, w.ctx_lens, 28, 4, 128)
    p0 = w.page_tables[0, 0]
    assert np.array_equal(got[0], np.repeat(v[p0, :, 0], 7, axis=0))      # ctx 1 -> o = V_0
    v[:] = 1.0
    got = run_attn(q, k, v, w.page_tables, w.ctx_lens, 28, 4, 128)
    assert np.all(got == np.float16(1.0))                                   # V == 1 -> o = 1


def test_empty_context_and_invalid_pages_are_safe():
    """ctx 0 gives zeros; an out-of-range page id contributes nothing and is
    counted, the other sequences are unaffected."""
    sh = wl.QWEN7B
    w = wl.custom("bad", 65, sh, [40, 40], 0)
    q = w.attn_q()
    k, v = w.kv(0)
    ref = run_attn(q, k, v, w.page_tables, w.ctx_lens, 28, 4, 128)
    pt = w.page_tables.copy()
    pt[1, 1] = 10_000
    ctx = w.ctx_lens.copy()
    got = run_attn(q, k, v, pt, ctx, 28, 4, 128)
    assert np.array_equal(got[0].view(np.uint16), ref[0].view(np.uint16))
    got = run_attn(q, k, v, w.page_tables, np.array([0, 40], np.int32), 28, 4, 128)
    assert np.all(got[0] == 0)
    assert np.array_equal(got[1].view(np.uint16), ref[1].view(np.uint16))


def fixed_pages_per_split(batch, n_kv, max_pages):
    """The launcher's fixed split size (pages): one page per wavefront until
    about 256 workgroups, at most 32 pages per wavefront, at most 128 splits."""
    units, pw = batch * n_kv * max_pages, 1
    while pw < 32 and units // (8 * pw) > 256:
        pw *= 2
    pps = 8 * pw
    while -(-max_pages // pps) > 128:
        pps *= 2
    return pps


@pytest.mark.parametrize("d,hq,hkv,ctx,width", [
    (128, 28, 4, [1, 17, 300, 3000, 2500, 16, 1200, 129], 4096),   # a few sequences, uneven
    (64, 7, 1, "u64", 512),                                         # 64 sequences
    (128, 16, 2, [5000, 10, 7000], 8192),                           # GQ 8
    (64, 8, 4, "u64", 1024),                                        # GQ 2, 256 (sequence, KV head) pairs
    (64, 8, 8, "u64", 1024),                                        # 512 pairs
    (128, 7, 1, [20000, 16], 16384),                                # a long sequence beside a short one
])
def test_uneven_contexts_in_long_splits(d, hq, hkv, ctx, width):
    """Page tables padded with -1 to `width` columns set the split size to
    16-32 pages per wavefront (first page issued early, default K/V load
    policy) while the contexts stay short enough for the oracle: most
    sequences end inside their first split, several wavefronts of a split
    have no page, a long one spans splits. A second call on the same
    workspace must give the same bits (the merging workgroup resets its
    arrival counter), and sequences whose context is then set to 0 give
    zeros while the others still match."""
    if isinstance(ctx, str):
        ctx = wl.rng(67, hq, width).integers(1, 2000, 64)
    ctx = np.asarray(ctx, np.int32)
    assert 1 < len(ctx) <= 64 and fixed_pages_per_split(len(ctx), hkv, width) >= 128
    sh = wl.Shape(hidden=hq * d, n_heads=hq, n_kv_heads=hkv, head_dim=d, ffn=8, vocab=8, n_layers=1)
    w = wl.custom("longsplit", 68 + hkv, sh, ctx)
    q = w.attn_q()
    k, v = w.kv(0)
    poison(k, v, w.page_tables, w.ctx_lens)
    pt = np.full((len(ctx), width), -1, np.int32)
    pt[:, :w.page_tables.shape[1]] = w.page_tables
    print(f"long-split attention d={d} heads={hq}/{hkv} batch={len(ctx)} width={width} "
          f"ctx {ctx.min()}..{ctx.max()}", flush=True)
    qd, kd, vd = to_dev(q), to_dev(k_pages_device(k)), to_dev(v_pages_device(v))
    ptd = torch.from_numpy(pt).cuda()
    cd = torch.from_numpy(ctx.copy()).cuda()
    ws = torch.empty(w4.paged_attention_workspace_bytes(len(ctx), hq, hkv, d, width), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((len(ctx), hq, d), dtype=torch.float16, device="cuda")
    call = lambda: w4.paged_attention_decode(qd, kd, vd, ptd, cd, hq, hkv, d, k.shape[0], ws, out)
    call()
    torch.cuda.synchronize()
    got = to_np16(out)
    ref = runs.attention_batch(w, q, k, v)
    assert_close(got, ref, f"long splits d={d} gqa={hq // hkv}")
    call()
    torch.cuda.synchronize()
    assert np.array_equal(to_np16(out).view(np.uint16), got.view(np.uint16)), "second call differs"
    zero = np.arange(len(ctx)) % 3 == 1
    cd.copy_(torch.from_numpy(np.where(zero, 0, ctx).astype(np.int32)))
    call()
    torch.cuda.synchronize()
    got2 = to_np16(out)
    assert np.all(got2[zero] == 0)
    assert_close(got2[~zero], ref[~zero], "long splits, some contexts empty")
