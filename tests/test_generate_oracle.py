"""Pins of the oracle's greedy generation loop ("Building a Custom LLM
Inference Runtime on H100", Architecture Overview: the token loop around the
decode step; "The Three Critical Bugs", Bug 1: position t in page t // 16,
slot t % 16) against hand examples and a dense brute-force loop."""
import math

import numpy as np
import pytest

import workloads as wl
from oracle import decode as od
from oracle import dense
from oracle import generate as og

TINY_LM = wl.Shape(hidden=200, n_heads=4, n_kv_heads=2, head_dim=16, ffn=72, vocab=96, n_layers=2)


@pytest.mark.parametrize("row,want", [
    ([1.0, 3.0, 3.0, 2.0], 1),                      # equal maxima: lowest index
    ([-np.inf, -np.inf, -np.inf], 0),               # all -inf: still a choice
    ([np.nan, 2.0, np.nan, 2.0], 1),                # NaN skipped
    ([np.nan, np.nan], -1),                         # nothing to choose
    ([1.0, float(np.float16(1.0) + np.finfo(np.float16).eps), 1.0], 1),   # one fp16 ulp apart
    ([-5.0], 0),
    ([0.0, -0.0], 0),                               # +0 == -0: lowest index
])
def test_greedy_token_hand_examples(row, want):
    assert og.greedy_token(np.array(row)) == want


def dense_generation(w, n_steps):
    """The same loop restated densely: contiguous per-head K/V histories that
    grow by appending, dense dequantised weights, dense lm_head, np.argmax."""
    sh, B = w.shape, w.batch
    p0 = w.ctx_lens - n_steps
    hist = {}
    for l in range(sh.n_layers):
        kp, vp = (a.astype(np.float64) for a in w.kv(l))
        for b in range(B):
            hk = np.stack([od.gather_kv(kp, w.page_tables[b], int(p0[b]), j) for j in range(sh.n_kv_heads)])
            hv = np.stack([od.gather_kv(vp, w.page_tables[b], int(p0[b]), j) for j in range(sh.n_kv_heads)])
            hist[l, b] = [hk, hv]
    w_lm = np.concatenate([wl.lm_head_chunk(w.workload_id, sh, c) for c in range(wl.n_chunks(sh))]).astype(np.float64)
    gamma_f = w.final_norm().astype(np.float64)
    tokens = w.tokens()
    toks, logits_all = [], []
    for s in range(n_steps):
        row_tok, row_logits = [], []
        for b in range(B):
            x = wl.embedding_rows(w.workload_id, sh, np.array([tokens[b]]))[0].astype(np.float64)
            for l in range(sh.n_layers):
                hk, hv = hist[l, b]
                x, kn, vn = dense.dense_layer(x, w.layer(l), hk, hv, int(p0[b]) + s, sh)
                hist[l, b] = [np.concatenate([hk, kn[:, None]], axis=1), np.concatenate([hv, vn[:, None]], axis=1)]
            logits = w_lm @ dense.rms(x, gamma_f, sh.eps)
            row_tok.append(int(np.argmax(logits)))
            row_logits.append(logits)
        toks.append(row_tok)
        logits_all.append(row_logits)
        tokens = np.array(row_tok)
    return np.array(toks), np.array(logits_all)


def test_generation_matches_dense_loop_across_page_boundaries():
    """Exact mode: two sequences, 20 steps each, starting at positions 11 and
    28, so both cross page boundaries (16, 32, 48) during the loop; the paged
    oracle's tokens and logits equal the dense loop's."""
    n = 20
    w = wl.custom("gen_tiny", 95, TINY_LM, [11 + n, 28 + n], layers=2, lm_head=True, gamma="random")
    got = og.generate(w, n, exact=True)
    toks, logits = dense_generation(w, n)
    assert np.allclose(got["logits"], logits, rtol=1e-9, atol=1e-9)
    assert np.array_equal(got["tokens"], toks)
    assert np.array_equal(got["positions"][:, 0], 11 + np.arange(n))
    assert len(set(got["tokens"][:, 0])) > 1          # the loop really feeds tokens back


def test_teacher_forcing_with_own_tokens_reproduces_the_free_run():
    n = 6
    w = wl.custom("gen_tiny", 96, TINY_LM, [30 + n], layers=2, lm_head=True, gamma="random")
    free = og.generate(w, n)
    forced = og.generate(w, n, forced=free["tokens"])
    assert np.array_equal(free["tokens"], forced["tokens"])
    assert np.array_equal(free["logits"], forced["logits"])
    # a different forced token changes every later step, not the first
    other = free["tokens"].copy()
    other[0, 0] = (other[0, 0] + 1) % TINY_LM.vocab
    alt = og.generate(w, n, forced=other)
    assert np.array_equal(alt["logits"][0], free["logits"][0])
    assert not np.array_equal(alt["logits"][1], free["logits"][1])


def test_generated_logits_are_fp16_values():
    w = wl.custom("gen_tiny", 97, TINY_LM, [5], layers=2, lm_head=True)
    got = og.generate(w, 3)
    lg = got["logits"]
    assert np.array_equal(lg, lg.astype(np.float16).astype(np.float64))
    assert all(math.isfinite(v) for v in lg.ravel())
