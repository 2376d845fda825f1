"""Greedy generation over the oracle decode step (test infrastructure only;
see the package header: only tests, the smoke check and the benchmark's CPU
baseline may use it).

Sources (page title, section):
  * "Building a Custom LLM Inference Runtime on H100", Architecture Overview:
    an orchestrator runs the token loop around the decode step, each step's
    output token being the next step's input.
  * Same page, "The Three Critical Bugs", Bug 1: a logical token position t
    lives in physical page page_table[t // 16] at slot t % 16, so a sequence
    needs a new page exactly when its position reaches a multiple of 16.

Readings where the pages are silent:
  * greedy choice = the token with the largest logit as stored (fp16); among
    equal maxima the lowest token id; NaN is never chosen (a row of NaNs has
    no choice, -1).
  * the loop starts from a workload whose page tables already cover the final
    context: sequence b decodes positions p0_b .. p0_b + n - 1 with
    p0_b = ctx_lens[b] - n, its first input token is the workload's token and
    its prior tokens [0, p0_b) are the workload's N(0,1) K/V. Pages beyond the
    prior context hold values that every step overwrites before reading, so
    which physical pages a real allocator would hand out does not change any
    result (paged attention is invariant under page permutations).
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

import workloads as wl
from . import decode as od
from . import runs


def greedy_token(row: np.ndarray) -> int:
    """Index of the largest value of `row`, the lowest index among equal
    maxima, NaN skipped; -1 if every value is NaN."""
    row = np.asarray(row, dtype=np.float64)
    ok = ~np.isnan(row)
    if not ok.any():
        return -1
    best = row[ok].max()
    return int(np.flatnonzero(row == best)[0])


def generate(w: "wl.Workload", n_steps: int, forced: Optional[np.ndarray] = None,
             exact: bool = False) -> Dict[str, np.ndarray]:
    """n_steps greedy decode steps for every sequence of `w` (a workload with
    an lm_head, contexts = the final contexts).

    forced: optional int [n_steps, B]; when given, the input of step s + 1 is
    forced[s] instead of the oracle's own choice (teacher forcing: the chosen
    tokens are still returned). Returns {"tokens": int [n_steps, B],
    "logits": float64 [n_steps, B, V], "positions": int [n_steps, B], "pools":
    the float64 (K, V) pools of every layer after the last step}.
    """
    sh, B = w.shape, w.batch
    assert w.lm_head and n_steps >= 1
    p0 = w.ctx_lens.astype(np.int64) - n_steps
    assert (p0 >= 0).all()
    weights = [w.layer(l) for l in range(sh.n_layers)]
    pools = [runs.pools_f64(w, l) for l in range(sh.n_layers)]
    gamma_f = w.final_norm()
    tokens = w.tokens().astype(np.int64)
    out_tok = np.zeros((n_steps, B), dtype=np.int64)
    out_logits = np.zeros((n_steps, B, sh.vocab))
    out_pos = np.zeros((n_steps, B), dtype=np.int64)
    for s in range(n_steps):
        pos = p0 + s
        x = wl.embedding_rows(w.workload_id, sh, tokens).astype(np.float64)
        for l in range(sh.n_layers):
            kp, vp = pools[l]
            for b in range(B):
                x[b] = od.decode_layer(x[b], weights[l], kp, vp, w.page_tables[b], int(pos[b]) + 1,
                                       sh, exact)
        xf = np.stack([od.rmsnorm(x[b], gamma_f, sh.eps, exact) for b in range(B)])
        logits = runs.lm_head_rows(w, xf, exact=exact)
        out_logits[s] = logits
        out_pos[s] = pos
        out_tok[s] = [greedy_token(logits[b]) for b in range(B)]
        tokens = np.asarray(forced[s], dtype=np.int64) if forced is not None else out_tok[s]
    return {"tokens": out_tok, "logits": out_logits, "positions": out_pos, "pools": pools}
