"""Greedy token choice (w4_argmax_f16) and the generation loop
(w4_generate_greedy) against the oracle ("Building a Custom LLM Inference
Runtime on H100", Architecture Overview: the token loop around the decode
step; "The Three Critical Bugs", Bug 1: positions mapped to pages as the
sequence grows)."""
import numpy as np
import pytest
import torch

import w4a16_paged_kv_amd as w4
import workloads as wl
from oracle import generate as og
from tests.gpu_util import assert_close, to_np16
from tests.staged import kv_slot
from workloads.device import DeviceModel, to_dev

pytestmark = pytest.mark.gpu

SMALL = wl.Shape(hidden=448, n_heads=7, n_kv_heads=1, head_dim=64, ffn=1536, vocab=5000, n_layers=3)


def f16_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.float16).view(np.int16)).cuda().view(torch.float16)


def gpu_argmax(rows: np.ndarray) -> np.ndarray:
    batch = rows.shape[0]
    out = torch.full((batch,), -7, dtype=torch.int32, device="cuda")
    ws = torch.full((w4.w4_argmax_workspace_bytes(batch, rows.shape[1]),), 0x7f, dtype=torch.uint8, device="cuda")
    w4.w4_argmax_f16(f16_dev(rows), out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("batch,vocab", [(1, 152064), (16, 152064), (3, 5000), (4, 5003), (2, 7),
                                         (16, 1), (5, 1001), (2, 2047), (3, 2049), (2, 131077)])
def test_argmax_matches_oracle_bit_exactly(batch, vocab):
    """Ragged vocabularies (odd and non-multiple-of-8 rows take the unaligned
    path on every other row; one chunk, two chunks, 64 chunks with a short
    last one), planted ties (also across chunks), -inf rows, NaNs."""
    rs = np.random.default_rng(1000 + vocab + batch)
    rows = rs.standard_normal((batch, vocab)).astype(np.float16)
    for b in range(batch):
        kind = b % 5
        if kind == 1 and vocab > 2:            # equal maxima: the lower index wins
            i, j = sorted(rs.choice(vocab, 2, replace=False))
            rows[b, i] = rows[b, j] = np.float16(rows[b].max() + 1)
        elif kind == 2:
            rows[b] = -np.inf
        elif kind == 3 and vocab > 2:          # NaNs around a finite maximum
            rows[b, rs.choice(vocab, max(1, vocab // 3), replace=False)] = np.nan
            rows[b, rs.integers(vocab)] = np.float16(9.0)
        elif kind == 4:
            rows[b, -1] = np.float16(100.0)    # maximum in the last (tail) element
    want = np.array([og.greedy_token(r.astype(np.float64)) for r in rows])
    assert np.array_equal(gpu_argmax(rows), want)


def test_argmax_all_nan_row_yields_minus_one():
    rows = np.full((2, 300), np.nan, dtype=np.float16)
    rows[1, 17] = 0.5
    assert list(gpu_argmax(rows)) == [-1, 17]


def setup_generation(w, p0, pool_pages=None):
    """DeviceModel of `w` plus a pool whose sequences already hold their prior
    tokens: the device KV cache is rearranged so that the pool's pages carry
    the workload's prior K/V."""
    dm = DeviceModel(w)
    pool = w4.KvPool(pool_pages or w.num_pages, w.batch)
    for b in range(w.batch):
        pool.kv_seq_reserve(b, int(p0[b]))
    pt0 = pool.page_table(list(range(w.batch)), w.max_pages)
    old = dm.kv_cache.clone()
    for b in range(w.batch):
        for i in range((int(p0[b]) + 15) // 16):
            dm.kv_cache[:, :, int(pt0[b, i])] = old[:, :, int(w.page_tables[b, i])]
    torch.cuda.synchronize()
    return dm, pool


def run_generation(dm, pool, w, p0, n, graph=True):
    dm.model.w4_set_graph(graph)
    logits = torch.empty((w.batch, w.shape.vocab), dtype=torch.float16, device="cuda")
    nxt = torch.empty((w.batch,), dtype=torch.int32, device="cuda")
    toks = dm.model.w4_generate_greedy(pool, list(range(w.batch)), w.tokens(), p0, n, logits, nxt)
    torch.cuda.synchronize()
    return toks, to_np16(logits)


@pytest.mark.parametrize("starts,n,wid", [([29, 13], 20, 31), ([0, 16, 5], 18, 33), ([29], 20, 34)])
def test_generation_matches_oracle(starts, n, wid):
    """20 steps from positions 29 and 13 (pages grow at 32, 48 and 16, 32),
    or 18 steps of three sequences: one with no prior context (its first page
    is reserved by the first step), one starting exactly on a page boundary,
    one mid-page, or one sequence alone. The pool ends exactly full. Teacher-forced with the GPU's
    tokens, the oracle confirms every choice: the chosen token's oracle logit is
    the maximum up to the logits' tolerance, and it is the oracle's own argmax
    wherever the oracle's top two are further apart than that. The last
    step's logits and every generated K/V slot of layer 0 are checked against
    the oracle; an eager rerun gives the same tokens and bit-identical logits."""
    p0 = np.array(starts, dtype=np.int32)
    print(f"generation from {starts}, {n} steps", flush=True)
    w = wl.custom("gen_small", wid, SMALL, p0 + n, layers=3, lm_head=True, gamma="random")
    dm, pool = setup_generation(w, p0)
    toks, last = run_generation(dm, pool, w, p0, n)
    print("generated", toks.T.tolist())
    assert ((toks >= 0) & (toks < SMALL.vocab)).all()
    for b in range(w.batch):
        assert pool.kv_seq_pages(b) == (int(p0[b]) + n + 15) // 16
    assert pool.kv_free_count() == 0

    ref = og.generate(w, n, forced=toks)
    agree = 0
    for s in range(n):
        for b in range(w.batch):
            L = ref["logits"][s, b]
            g = int(toks[s, b])
            order = np.argsort(-L, kind="stable")
            top, second = L[order[0]], L[order[1]]
            e = 2e-3 + 1e-2 * max(abs(top), float(np.sqrt((L ** 2).mean())))
            assert L[g] >= top - 2 * e, f"step {s} seq {b}: token {g} logit {L[g]} vs max {top}"
            if top - second > 2 * e:
                assert g == int(order[0]), f"step {s} seq {b}: clear argmax {order[0]} not chosen"
            agree += g == ref["tokens"][s, b]
    print(f"{agree} of {n * w.batch} choices equal the oracle's own argmax")

    L = ref["logits"][-1]
    err = np.abs(last.astype(np.float64) - L)
    ok = err <= 2e-3 + 1e-2 * np.abs(L)
    assert ok.mean() > 0.99
    assert err.max() < 1e-2 * np.sqrt((L ** 2).mean())

    ptf = pool.page_table(list(range(w.batch)), w.max_pages)
    kp, vp = ref["pools"][0]
    for b in range(w.batch):
        for pos in range(int(p0[b]), int(p0[b]) + n):
            page_g, page_o, slot = int(ptf[b, pos // 16]), int(w.page_tables[b, pos // 16]), pos % 16
            assert_close(kv_slot(dm, 0, 0, page_g, slot), kp[page_o, :, slot], f"seq {b} pos {pos}: k")
            assert_close(kv_slot(dm, 0, 1, page_g, slot), vp[page_o, :, slot], f"seq {b} pos {pos}: v")

    pool2 = w4.KvPool(w.num_pages, w.batch)
    for b in range(w.batch):
        pool2.kv_seq_reserve(b, int(p0[b]))
    toks2, last2 = run_generation(dm, pool2, w, p0, n, graph=False)
    assert np.array_equal(toks, toks2)
    assert np.array_equal(last.view(np.uint16), last2.view(np.uint16))


def test_generation_errors():
    n = 4
    p0 = np.array([14], dtype=np.int32)
    w = wl.custom("gen_small", 32, SMALL, p0 + n, layers=3, lm_head=True)
    dm, pool = setup_generation(w, p0, pool_pages=1)   # the prior page only: growth at 16 fails
    logits = torch.empty((1, SMALL.vocab), dtype=torch.float16, device="cuda")
    nxt = torch.empty((1,), dtype=torch.int32, device="cuda")
    assert dm.model.w4_generate_greedy(pool, [0], w.tokens(), p0, 0, logits, nxt).shape == (0, 1)
    with pytest.raises(w4.W4Error, match="ENOPAGES"):
        dm.model.w4_generate_greedy(pool, [0], w.tokens(), p0, n, logits, nxt)
    with pytest.raises(w4.W4Error, match="ERANGE"):      # positions beyond 16 * max_pages
        dm.model.w4_generate_greedy(pool, [0], w.tokens(), [16 * w.max_pages - 1], 2, logits, nxt)
    with pytest.raises(w4.W4Error, match="ERANGE"):      # prior tokens not held by the sequence
        dm.model.w4_generate_greedy(pool, [0], w.tokens(), [20], 1, logits, nxt)
    with pytest.raises(w4.W4Error, match="ERANGE"):      # first token outside the vocabulary
        dm.model.w4_generate_greedy(pool, [0], [SMALL.vocab], p0, 1, logits, nxt)
    torch.cuda.synchronize()


def test_generation_full_size_matches_decode_step():
    """The 28-layer Qwen2.5-7B-shape model, batch 1, the loop as the benchmark
    runs it (start 16 tokens before the 2048-token context ends, so the pool
    grows at position 2032): after two steps the logits equal a separate
    decode_step of the second step's inputs bit for bit, the chosen tokens
    are the host argmax of those logits (lowest index), and the sequence
    holds 128 pages."""
    w = wl.step_b1()
    print("building the 28-layer model", flush=True)
    dm = DeviceModel(w)
    p0 = (w.ctx_lens - 16).astype(np.int32)
    pool = w4.KvPool(w.num_pages, 1)
    pool.kv_seq_reserve(0, int(p0[0]))
    assert pool.kv_seq_pages(0) == 127
    toks, last = run_generation(dm, pool, w, p0, 2)
    assert pool.kv_seq_pages(0) == 128
    assert og.greedy_token(last[0].astype(np.float64)) == toks[1, 0]
    pt = pool.page_table([0], w.max_pages)
    logits = torch.empty((1, w.shape.vocab), dtype=torch.float16, device="cuda")
    dm.model.decode_step(toks[0], p0 + 1, pt, p0 + 2, logits)
    torch.cuda.synchronize()
    again = to_np16(logits)
    assert np.array_equal(again.view(np.uint16), last.view(np.uint16))
    assert dm.model.w4_device_errors() == 0


def test_generation_skips_nan_logits_and_stops_on_all_nan():
    """Through the generation loop (batch 1): lm_head rows set to NaN (every
    third row and the previously chosen one) give NaN logits that are never
    chosen (the choice equals the oracle's rule on the step's own logits), and
    with every row NaN the loop stops with W4_ERANGE before a second step,
    next_tokens reading -1."""
    from workloads import lm_head_chunk, n_chunks
    p0 = np.array([21], dtype=np.int32)
    w = wl.custom("gen_nan", 35, SMALL, p0 + 2, layers=3, lm_head=True, gamma="random")
    dm, pool = setup_generation(w, p0)
    sh = w.shape
    W = np.concatenate([lm_head_chunk(w.workload_id, sh, c) for c in range(n_chunks(sh))])
    toks, last = run_generation(dm, pool, w, p0, 1)
    best = og.greedy_token(last[0].astype(np.float64))
    assert toks[0, 0] == best
    Wn = W.copy()
    nan_rows = np.unique(np.concatenate([[best], np.arange(0, sh.vocab, 3)]))
    Wn[nan_rows] = np.nan                        # the previous best among them
    dm.lm_head.copy_(to_dev(w4.pack_weights_f16(Wn)).view(torch.uint8).view(-1))
    pool2 = w4.KvPool(w.num_pages, 1)
    pool2.kv_seq_reserve(0, int(p0[0]))
    toks2, last2 = run_generation(dm, pool2, w, p0, 1)
    assert np.isnan(last2[0, nan_rows]).all() and not np.isnan(np.delete(last2[0], nan_rows)).any()
    assert toks2[0, 0] == og.greedy_token(last2[0].astype(np.float64)) and toks2[0, 0] not in nan_rows
    Wn[:] = np.nan
    dm.lm_head.copy_(to_dev(w4.pack_weights_f16(Wn)).view(torch.uint8).view(-1))
    pool3 = w4.KvPool(w.num_pages, 1)
    pool3.kv_seq_reserve(0, int(p0[0]))
    logits = torch.empty((1, sh.vocab), dtype=torch.float16, device="cuda")
    nxt = torch.empty((1,), dtype=torch.int32, device="cuda")
    with pytest.raises(w4.W4Error, match="every logit is NaN") as e:
        dm.model.w4_generate_greedy(pool3, [0], w.tokens(), p0, 2, logits, nxt)
    assert e.value.steps_done == 0
    torch.cuda.synchronize()
    assert int(nxt.cpu()[0]) == -1
    assert dm.model.w4_device_errors() == 0
