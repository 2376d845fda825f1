"""Planted mistakes in the CPU oracle must each fail at least one pin.

Every mutation below replaces one oracle function with a copy that makes a
plausible mistake (a dropped term, a wrong sign or index, a rounding in the
wrong place). The pins of tests/test_oracle_pins.py are then run against the
mutated oracle; the stored-output golden is left out, because it was written
by the oracle itself and would only show that something changed. A mutation
that no other pin catches marks a gap in the pins.

Everything here runs on the CPU and touches only the oracle.
"""
import inspect
import math

import numpy as np
import pytest

from oracle import decode as od
from tests import test_oracle_pins as pins

R = od.r16


def _pin_calls():
    """(name, callable) for every pin, one per parameter set."""
    out = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_") or name == "test_oracle_reproduces_its_stored_layer_output":
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not marks:
            out.append((name, fn))
            continue
        argnames, values = marks[0].args
        argnames = [a.strip() for a in argnames.split(",")]
        for vals in values:
            vals = vals if len(argnames) > 1 else (vals,)
            out.append((f"{name}{list(vals)}", lambda fn=fn, kw=dict(zip(argnames, vals)): fn(**kw)))
    return out


def _failing_pins():
    failed = []
    with np.errstate(all="ignore"):
        for name, call in _pin_calls():
            try:
                call()
            except (Exception, pytest.fail.Exception):   # an assertion, a wrong shape, a missed raise
                failed.append(name)
    return failed


# --------------------------------------------------------------- mutations

def _split_qkv_rounding_q_first(orig):
    return lambda y, w, pos, sh, exact, mirror=False: orig(y, w, pos, sh, exact, True)


def _gate_up_rounding_first(orig):
    return lambda xn2, w, shape, exact=False, mirror=False: orig(xn2, w, shape, exact, True)


def _split_qkv_v_unrounded(orig):
    def f(y, w, pos, sh, exact, mirror=False):
        q, k, _ = orig(y, w, pos, sh, exact, mirror)
        yb = y + (0 if w.qkv_bias is None else np.asarray(w.qkv_bias, np.float64))
        return q, k, yb[sh.q_rows + sh.kv_rows:].reshape(sh.n_kv_heads, sh.head_dim)
    return f


def _oproj_double_round(orig):
    return lambda x, o, w, exact=False: R(np.asarray(x, np.float64) + R(od.gemv_w4(
        w.o_q, w.o_s, np.asarray(o, np.float64).reshape(np.shape(x)[:-1] + (-1,)), ), exact), exact)


def _down_double_round(orig):
    return lambda x1, h, w, exact=False: R(np.asarray(x1, np.float64) + R(od.gemv_w4(
        w.down_q, w.down_s, np.asarray(h, np.float64)), exact), exact)


def _rmsnorm_double_round(orig):
    def f(x, gamma, eps, exact=False):
        x = np.asarray(x, np.float64)
        ms = (x * x).sum(axis=-1, keepdims=True) / x.shape[-1]
        return R(R(x / np.sqrt(ms + eps), exact) * np.asarray(gamma, np.float64), exact)
    return f


def _rmsnorm_sum_not_mean(orig):
    def f(x, gamma, eps, exact=False):
        x = np.asarray(x, np.float64)
        ms = (x * x).sum(axis=-1, keepdims=True)
        return R(x / np.sqrt(ms + eps) * np.asarray(gamma, np.float64), exact)
    return f


def _attention(kv_head_of, scale_of):
    def f(q, k_pool, v_pool, page_table_row, ctx, exact=False):
        q = np.asarray(q, np.float64)
        hq, d = q.shape
        hkv = k_pool.shape[1]
        out = np.empty((hq, d))
        for h in range(hq):
            j = kv_head_of(h, hq, hkv)
            kj = od.gather_kv(k_pool, page_table_row, ctx, j)
            vj = od.gather_kv(v_pool, page_table_row, ctx, j)
            out[h] = od.softmax(kj @ q[h] * scale_of(d)) @ vj
        return R(out, exact)
    return lambda orig: f


def _page_slot(page_of, slot_of):
    return lambda orig: (lambda row, t: (int(row[page_of(t)]), slot_of(t)))


def _rope(sign, two):
    def f(v, pos, base, exact=False):
        v = np.asarray(v, np.float64)
        half = v.shape[-1] // 2
        i = np.arange(half, dtype=np.float64)
        th = float(pos) * np.power(float(base), -two * i / v.shape[-1])
        c, s = np.cos(th), sign * np.sin(th)
        a, b = v[..., :half], v[..., half:]
        return R(np.concatenate([a * c - b * s, b * c + a * s], axis=-1), exact)
    return lambda orig: f


def _dequant_group(g):
    def f(q, s):
        n, k = q.shape
        sk = np.repeat(np.asarray(s, np.float64), g, axis=1)
        sk = np.pad(sk, ((0, 0), (0, max(0, k - sk.shape[1]))), mode="edge")[:, :k]
        return q.astype(np.float64) * sk
    return lambda orig: f


def _silu_sign(orig):
    return lambda z: np.asarray(z, np.float64) / (1.0 + np.exp(np.asarray(z, np.float64)))


def _gate_up_swapped(orig):
    def f(xn2, w, shape, exact=False, mirror=False):
        gu = od.gemv_w4(w.gate_up_q, w.gate_up_s, np.asarray(xn2, np.float64))
        g, u = gu[..., shape.ffn:], gu[..., :shape.ffn]
        return R(od.silu(g) * u, exact)
    return f


def _oproj_no_residual(orig):
    return lambda x, o, w, exact=False: R(od.gemv_w4(
        w.o_q, w.o_s, np.asarray(o, np.float64).reshape(np.shape(x)[:-1] + (-1,))), exact)


def _layer_variant(write_after_attention=False, pos_shift=0, rope_v=False):
    def f(x, w, k_pool, v_pool, pt, ctx, shape, exact=False, mirror=False):
        pos = ctx - 1 + pos_shift
        q, k, v = od.qkv_stage(x, w, pos, shape, exact, mirror)
        if rope_v:
            v = od.rope(v, pos, shape.rope_base, exact)
        if not write_after_attention:
            od.kv_write(k_pool, v_pool, pt, ctx - 1, k, v)
        o = od.attention_decode(q, k_pool, v_pool, pt, ctx, exact)
        if write_after_attention:
            od.kv_write(k_pool, v_pool, pt, ctx - 1, k, v)
        x1 = od.oproj_stage(x, o, w, exact)
        h = od.gate_up_stage(x1, w, shape, exact, mirror)
        return od.down_stage(x1, h, w, exact)
    return lambda orig: f


MUTATIONS = {
    # rounding placement
    "q and k rounded before RoPE": ("_split_qkv", _split_qkv_rounding_q_first),
    "gate and up rounded before SiLU": ("gate_up_from_normed", _gate_up_rounding_first),
    "v left unrounded": ("_split_qkv", _split_qkv_v_unrounded),
    "o-projection residual rounded twice": ("oproj_stage", _oproj_double_round),
    "down-projection residual rounded twice": ("down_stage", _down_double_round),
    "RMSNorm rounded before gamma": ("rmsnorm", _rmsnorm_double_round),
    # arithmetic and indexing
    "RMSNorm over the sum, not the mean": ("rmsnorm", _rmsnorm_sum_not_mean),
    "GQA heads interleaved (h % Hkv)": ("attention_decode", _attention(lambda h, hq, hkv: h % hkv,
                                                                      lambda d: 1 / math.sqrt(d))),
    "scores not scaled by 1/sqrt(D)": ("attention_decode", _attention(lambda h, hq, hkv: h // (hq // hkv),
                                                                     lambda d: 1.0)),
    "slot off by one": ("page_slot", _page_slot(lambda t: t // 16, lambda t: (t + 1) % 16)),
    "page off by one": ("page_slot", _page_slot(lambda t: (t + 1) // 16, lambda t: t % 16)),
    "RoPE turning the wrong way": ("rope", _rope(-1.0, 2.0)),
    "RoPE exponent -i/D": ("rope", _rope(1.0, 1.0)),
    "scale groups of 64": ("dequant_w4g128", _dequant_group(64)),
    "SiLU sign": ("silu", _silu_sign),
    "gate and up swapped": ("gate_up_from_normed", _gate_up_swapped),
    "residual dropped": ("oproj_stage", _oproj_no_residual),
    "K/V written after attention": ("decode_layer", _layer_variant(write_after_attention=True)),
    "position = ctx, not ctx - 1": ("decode_layer", _layer_variant(pos_shift=1)),
    "RoPE applied to v": ("decode_layer", _layer_variant(rope_v=True)),
}


def test_unmutated_oracle_passes_every_pin():
    assert _failing_pins() == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_fails_a_pin(name, monkeypatch):
    attr, make = MUTATIONS[name]
    monkeypatch.setattr(od, attr, make(getattr(od, attr)))
    failed = _failing_pins()
    assert failed, f"no pin catches the mutation '{name}'"
    print(f"{name}: caught by {len(failed)} pins, e.g. {failed[:3]}")
