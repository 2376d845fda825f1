"""Pins of the oracle's prefill (CPU only): a prompt run through the model at
once must equal the same prompt decoded one token at a time by the decode
oracle (itself pinned against the dense brute force), in the last token's
logits, every prompt row's residual and every K/V slot written -- with and
without prior context in the pages ("How to build your own LLM runtime from
scratch", Key performance metrics: time to first token of a 512-token
prompt; "Building a Custom LLM Inference Runtime on H100", The KV Cache and
PagedAttention)."""
import numpy as np
import pytest

import workloads as wl
from oracle import decode as od
from oracle import prefill as op
from oracle import runs

SHAPE = wl.Shape(hidden=256, n_heads=7, n_kv_heads=1, head_dim=32, ffn=136, vocab=300, n_layers=2)
SHAPE4 = wl.Shape(hidden=200, n_heads=4, n_kv_heads=2, head_dim=16, ffn=72, vocab=97, n_layers=2)


def sequential(w, tokens, start, exact):
    """The prompt decoded token by token: each token through every layer, its
    K/V written before the next token starts."""
    sh = w.shape
    pools = [runs.pools_f64(w, l) for l in range(sh.n_layers)]
    weights = [w.layer(l) for l in range(sh.n_layers)]
    rows = []
    for i, tok in enumerate(tokens):
        x = wl.embedding_rows(w.workload_id, sh, np.array([tok]))[0].astype(np.float64)
        for l in range(sh.n_layers):
            kp, vp = pools[l]
            x = od.decode_layer(x, weights[l], kp, vp, w.page_tables[0], start + i + 1, sh, exact)
        rows.append(x)
    xf = od.rmsnorm(rows[-1][None], w.final_norm(), sh.eps, exact)
    return runs.lm_head_rows(w, xf, exact=exact)[0], np.stack(rows), pools


@pytest.mark.parametrize("shape,start,n", [(SHAPE, 0, 37), (SHAPE, 5, 12), (SHAPE4, 16, 17), (SHAPE4, 0, 1)])
@pytest.mark.parametrize("exact", [True, False])
def test_prefill_equals_token_by_token_decode(shape, start, n, exact):
    w = wl.custom("prefill_pin", 96, shape, [start + n], layers=shape.n_layers, lm_head=True, gamma="random")
    tokens = w.prompt_tokens(n)
    got = runs.prefill_run(w, tokens, start, exact=exact, keep_pools=True)
    ref_logits, ref_rows, ref_pools = sequential(w, tokens, start, exact)
    tol = dict(rtol=1e-10, atol=1e-10) if exact else dict(rtol=0, atol=0)
    assert np.allclose(got["logits"], ref_logits, **tol)
    assert np.allclose(got["x"], ref_rows, **tol)
    for (kp, vp), (kr, vr) in zip(got["pools"], ref_pools):
        assert np.allclose(kp, kr, **tol) and np.allclose(vp, vr, **tol)


def test_prefill_is_causal_and_writes_only_the_prompt_slots():
    """Changing the last prompt token changes no earlier row and no earlier
    K/V slot; slots outside [start, start + n) keep the pages' prior values."""
    w = wl.custom("prefill_causal", 97, SHAPE, [40], layers=2, lm_head=True, gamma="random")
    tokens = w.prompt_tokens(30)
    start = 10
    a = runs.prefill_run(w, tokens, start, keep_pools=True)
    t2 = tokens.copy()
    t2[-1] = (t2[-1] + 1) % SHAPE.vocab
    b = runs.prefill_run(w, t2, start, keep_pools=True)
    assert np.array_equal(a["x"][:-1], b["x"][:-1]) and not np.array_equal(a["x"][-1], b["x"][-1])
    pt = w.page_tables[0]
    for l in range(2):
        k0, v0 = runs.pools_f64(w, l)
        for t in range(40):
            page, slot = pt[t // 16], t % 16
            if not start <= t < start + 30:       # outside the prompt: untouched
                assert np.array_equal(a["pools"][l][0][page, :, slot], k0[page, :, slot])
                assert np.array_equal(a["pools"][l][1][page, :, slot], v0[page, :, slot])
            if t < start + 29:                    # before the changed token: unaffected
                assert np.array_equal(a["pools"][l][0][page, :, slot], b["pools"][l][0][page, :, slot])
                assert np.array_equal(a["pools"][l][1][page, :, slot], b["pools"][l][1][page, :, slot])


def test_prefill_of_one_token_is_the_decode_step():
    """n = 1: prefill is exactly one decode step of that token."""
    w = wl.custom("prefill_one", 98, SHAPE4, [21], layers=2, lm_head=True, gamma="random")
    tok = w.prompt_tokens(1)
    got = runs.prefill_run(w, tok, 20)
    w1 = wl.Workload(w.name, w.workload_id, w.shape, 1, np.array([21], np.int32), w.page_tables, w.num_pages,
                     2, True, w.gamma)
    w1.tokens = lambda: tok
    ref = runs.step(w1)
    assert np.array_equal(got["logits"], ref["logits"][0])
