"""Pins of the CPU oracle against closed forms, invariants, hand-worked
examples and brute force -- none of them re-types the oracle's own formula.

Each test names the passage it follows; the pages themselves print no worked
numbers for any intermediate, so every pin here is mathematical.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import workloads as wl
from oracle import decode as od
from oracle import dense


def f16(x):
    return np.float16(x)


# ------------------------------------------------------------------ rounding

def test_r16_is_round_to_nearest_even():
    one = 1.0
    ulp = 2.0 ** -10
    assert od.r16(one + ulp / 2) == one                     # tie -> even (1.0)
    assert od.r16(one + 3 * ulp / 2) == one + 2 * ulp       # tie -> even mantissa
    assert od.r16(one + ulp / 2 + 2.0 ** -20) == one + ulp  # above the tie
    assert od.r16(70000.0) == np.inf
    assert od.r16(2.0 ** -25 + 2.0 ** -40) == 2.0 ** -24    # subnormal rounding


# ------------------------------------------------------------------ dequant

SPECIAL_SCALES = [0.0, 2.0 ** -24, 6.103515625e-05, 1.0, 65504.0,
                  float(f16(0.02 * 0.3)), float(f16(0.02 * 1.7)), float(f16(0.02 * 2.9))]


def test_dequant_closed_form_every_code_and_special_scales():
    """W = q * s exactly for all 16 codes and extreme fp16 scales
    ("How to build your own LLM runtime from scratch", Architectural
    decisions: symmetric group-wise INT4, group 128)."""
    q = np.tile(np.arange(-8, 8, dtype=np.int8), (len(SPECIAL_SCALES), 8))   # [8, 128]
    s = np.array(SPECIAL_SCALES, dtype=np.float16)[:, None]
    w = od.dequant_w4g128(q, s)
    for n in range(q.shape[0]):
        for k in range(q.shape[1]):
            exact = Fraction(int(q[n, k])) * Fraction(float(s[n, 0]))
            assert Fraction(w[n, k]) == exact


def test_dequant_group_axis_and_partial_group():
    """Groups of 128 run along the input columns; K = 448 has 3 full groups
    and one of 64 (the miniature layer's hidden size)."""
    n, k = 5, 448
    rs = np.random.default_rng(0)
    q = rs.integers(-8, 8, (n, k)).astype(np.int8)
    s = (np.arange(n * 4).reshape(n, 4) + 1).astype(np.float16)   # distinct per (row, group)
    w = od.dequant_w4g128(q, s)
    for nn in range(n):
        for kk in (0, 127, 128, 255, 256, 383, 384, 447):
            assert w[nn, kk] == int(q[nn, kk]) * float(s[nn, kk // 128])


def test_dequant_rejects_out_of_range_codes():
    with pytest.raises(AssertionError):
        od.dequant_w4g128(np.array([[8]], dtype=np.int8), np.ones((1, 1), np.float16))


# ------------------------------------------------------------------ GEMV

def test_gemv_one_hot_selects_a_column():
    rs = np.random.default_rng(1)
    q = rs.integers(-8, 8, (7, 300)).astype(np.int8)
    s = wl.group_scales(rs, 7, 300)
    for col in (0, 5, 127, 128, 299):
        x = np.zeros(300)
        x[col] = 1.0
        y = od.gemv_w4(q, s, x)
        assert np.array_equal(y, q[:, col].astype(np.float64) * s[:, col // 128].astype(np.float64))


def test_gemv_constant_codes_sum_to_c_times_k():
    for c in (-8, -3, 0, 7):
        q = np.full((3, 448), c, dtype=np.int8)
        s = np.ones((3, 4), dtype=np.float16)
        y = od.gemv_w4(q, s, np.ones(448))
        assert np.all(y == c * 448)


def test_gemv_matches_pure_python_loops():
    rs = np.random.default_rng(2)
    n, k = 4, 260
    q = rs.integers(-8, 8, (n, k)).astype(np.int8)
    s = wl.group_scales(rs, n, k)
    x = rs.standard_normal(k).astype(np.float16)
    y = od.gemv_w4(q, s, x, rows_per_chunk=3)
    for i in range(n):
        acc = math.fsum(int(q[i, j]) * float(s[i, j // 128]) * float(x[j]) for j in range(k))
        assert abs(y[i] - acc) <= 1e-12 * max(1.0, abs(acc))


# ------------------------------------------------------------------ RMSNorm

def test_rmsnorm_hand_example():
    """x = (3, 4): mean square 12.5, so y = x / sqrt(12.5 + eps) * gamma."""
    y = od.rmsnorm(np.array([3.0, 4.0]), np.array([1.0, 2.0]), 0.0, exact=True)
    assert y[0] == pytest.approx(3 / math.sqrt(12.5), rel=1e-15)
    assert y[1] == pytest.approx(8 / math.sqrt(12.5), rel=1e-15)


def test_rmsnorm_constant_vector_and_eps():
    for c in (0.5, 3.0, -7.25):
        x = np.full(448, c)
        y = od.rmsnorm(x, np.ones(448), 1e-6)
        expect = float(f16(c / math.sqrt(c * c + 1e-6)))
        assert np.all(y == expect)
    assert np.all(od.rmsnorm(np.zeros(8), np.ones(8), 1e-6) == 0.0)


def test_rmsnorm_scale_invariance():
    rs = np.random.default_rng(3)
    x = rs.standard_normal(3584)
    g = 1 + 0.1 * rs.standard_normal(3584)
    a = od.rmsnorm(x, g, 0.0, exact=True)
    b = od.rmsnorm(17.0 * x, g, 0.0, exact=True)
    assert np.allclose(a, b, rtol=1e-14, atol=0)


# ------------------------------------------------------------------ RoPE

def test_rope_position_zero_is_identity():
    v = np.random.default_rng(4).standard_normal(128).astype(np.float16)
    assert np.array_equal(od.rope(v, 0, 1e6), v.astype(np.float64))


def test_rope_hand_example_rotate_half_d4():
    """D = 4, base 1e6, pos 1: theta_0 = 1, theta_1 = 1e6^(-1/2) = 1e-3;
    pairs are (0, 2) and (1, 3)."""
    y = od.rope(np.array([1.0, 0.0, 0.0, 0.0]), 1, 1e6, exact=True)
    assert np.allclose(y, [math.cos(1), 0, math.sin(1), 0], rtol=0, atol=1e-15)
    y = od.rope(np.array([0.0, 1.0, 0.0, 0.0]), 1, 1e6, exact=True)
    assert np.allclose(y, [0, math.cos(1e-3), 0, math.sin(1e-3)], rtol=0, atol=1e-15)
    y = od.rope(np.array([0.0, 0.0, 0.0, 2.0]), 3, 1e6, exact=True)
    assert np.allclose(y, [0, -2 * math.sin(3e-3), 0, 2 * math.cos(3e-3)], rtol=0, atol=1e-15)


def test_rope_is_complex_rotation_and_relative():
    rs = np.random.default_rng(5)
    q = rs.standard_normal(128)
    k = rs.standard_normal(128)
    for pos in (1, 17, 511, 2047, 8191):
        assert np.allclose(od.rope(q, pos, 1e6, exact=True), dense.rotate(q, pos, 1e6), atol=1e-12)
        r = od.rope(q, pos, 1e6, exact=True)
        pair_norm = q[:64] ** 2 + q[64:] ** 2
        assert np.allclose(r[:64] ** 2 + r[64:] ** 2, pair_norm, rtol=1e-12)
    for m, n in ((5, 2), (100, 37), (2047, 2000)):
        lhs = od.rope(q, m, 1e6, exact=True) @ od.rope(k, n, 1e6, exact=True)
        rhs = od.rope(q, m - n, 1e6, exact=True) @ k
        assert abs(lhs - rhs) < 1e-10


# ------------------------------------------------------------------ SiLU

def test_silu_limits():
    assert od.silu(0.0) == 0.0
    assert abs(od.silu(40.0) - 40.0) < 1e-14
    assert abs(od.silu(-40.0)) < 1e-15
    assert od.silu(1.0) == pytest.approx(1 / (1 + math.exp(-1)), rel=1e-15)


# ------------------------------------------------------------------ rounding placement
# Where the fp16 roundings sit (RMSNorm and lm_head "kept in FP16", fp16
# activations: "How to build your own LLM runtime from scratch",
# Architectural decisions and optimizations). The reading: one rounding per
# stored tensor -- r(RMSNorm(x)) as a whole, v rounded, q and k rotated
# unrounded and rounded once after RoPE, gate and up unrounded before SiLU,
# h = r(silu(g) u), each residual add x + W y rounded once. Each hand example
# below has inputs chosen (exact binary fractions) so that moving one rounding
# changes the fp16 result; the expected values were worked out to 60 digits
# (decimal arithmetic, cos 1 and sin 1 by their series) and are written here
# as literals, with the value the other placement would give beside them.

def _hand_layer(hidden, qkv_rows=None, gate_up=None, o=None, down=None):
    """LayerWeights of a hand example: each given matrix as (codes, scales)."""
    z = lambda n, k: (np.zeros((n, k), np.int8), np.zeros((n, 1), np.float16))
    qkv = qkv_rows or z(6, hidden)
    gu = gate_up or z(2, hidden)
    oo = o or z(hidden, 2)
    dd = down or z(hidden, 2)
    one = np.ones(hidden, np.float16)
    return wl.LayerWeights(np.asarray(qkv[0], np.int8), np.asarray(qkv[1], np.float16),
                           np.asarray(oo[0], np.int8), np.asarray(oo[1], np.float16),
                           np.asarray(gu[0], np.int8), np.asarray(gu[1], np.float16),
                           np.asarray(dd[0], np.int8), np.asarray(dd[1], np.float16), one, one)


HAND = wl.Shape(hidden=2, n_heads=1, n_kv_heads=1, head_dim=2, ffn=1, vocab=1, n_layers=1)


def test_rounding_q_k_rotated_unrounded_v_rounded_once():
    """xn = (1, 2^-13). q = k = (a, b) with a = 1 + 5 2^-13 (not an fp16 value;
    r(a) = 1 + 2^-10) and b = 0.6416015625; v = (a, 2^-13). D = 2 and pos = 1,
    so the one RoPE pair turns by 1 radian: q'_0 = a cos 1 - b sin 1 =
    7.4292...e-4 cancels, and rounding a first would move it by ~400 ulps."""
    codes = [[1, 5], [1, 0], [1, 5], [1, 0], [1, 5], [0, 1]]
    scales = [[1.0], [0.6416015625], [1.0], [0.6416015625], [1.0], [1.0]]
    lw = _hand_layer(2, qkv_rows=(codes, scales))
    xn = np.array([1.0, 2.0 ** -13])
    q, k, v = od.qkv_from_normed(xn, lw, 1, HAND)
    rotated = [0.0007429122924804688, 1.1884765625]    # r(a cos1 - b sin1), r(b cos1 + a sin1)
    assert q.tolist() == [rotated] and k.tolist() == [rotated]
    assert v.tolist() == [[1.0009765625, 2.0 ** -13]]   # r(a) = 1 + 2^-10
    # the other placement (q, k rounded before RoPE) gives a different q'_0
    qm, km, vm = od.qkv_from_normed(xn, lw, 1, HAND, mirror=True)
    assert qm.tolist() == [[0.0009407997131347656, 1.1884765625]] and km.tolist() == qm.tolist()
    assert vm.tolist() == v.tolist()


def test_rounding_gate_and_up_unrounded_before_silu():
    """xn2 = (1.25, 2^-9); gate codes (-8, -6), up codes (6, 5), scales 1:
    g = -10.01171875 (r(g) = -10.015625), u = 7.509765625 (r(u) = 7.5078125).
    h = r(silu(g) u) with silu(g) = g / (1 + e^-g) = -4.4921...e-4."""
    lw = _hand_layer(2, gate_up=([[-8, -6], [6, 5]], [[1.0], [1.0]]))
    xn2 = np.array([1.25, 2.0 ** -9])
    h = od.gate_up_from_normed(xn2, lw, HAND)
    assert h.tolist() == [-0.0033740997314453125]
    # g rounded first: seven fp16 steps away (-0.003360748291015625); u
    # rounded first: one step (-0.0033721923828125); both rounded (the mirror)
    assert od.gate_up_from_normed(xn2, lw, HAND, mirror=True).tolist() == [-0.003360748291015625]


@pytest.mark.parametrize("stage", ["oproj", "down"])
def test_rounding_residual_add_rounds_once(stage):
    """x = 1, W y = 2^-11 + 2^-24 (codes (1, 1), scale 1, y = (2^-11, 2^-24)).
    One rounding of x + W y = 1 + 2^-11 + 2^-24 (just past the tie) gives
    1 + 2^-10; rounding W y first (to 2^-11) would leave a tie that rounds to
    even, 1.0."""
    w = ([[1, 1]], [[1.0]])
    lw = _hand_layer(1, o=w, down=w)
    x = np.array([1.0])
    y = np.array([2.0 ** -11, 2.0 ** -24])
    out = od.oproj_stage(x, y, lw) if stage == "oproj" else od.down_stage(x, y, lw)
    assert out.tolist() == [1.0009765625]


def test_rounding_rmsnorm_rounds_once():
    """x = (3, 4), eps = 0: x / rms = (3, 4) / sqrt(12.5) = (0.84852.., 1.13137..);
    times gamma = 0.513671875 and rounded once: (0.435791015625, 0.5810546875).
    Rounding x / rms first would give (0.43603515625, 0.58154296875)."""
    g = np.full(2, 0.513671875)
    assert od.rmsnorm(np.array([3.0, 4.0]), g, 0.0).tolist() == [0.435791015625, 0.5810546875]


def test_mirror_is_off_by_default_and_exact_mode_ignores_it():
    """mirror only adds roundings: in exact mode it changes nothing, and on a
    real layer the two placements stay within a few fp16 steps of each other."""
    w = wl.custom("mirror", 92, TINY7, [40], gamma="random")
    lw = w.layer(0, bias=True)
    x = w.x_in()[0].astype(np.float64)
    outs = {}
    for exact in (True, False):
        for mirror in (False, True):
            kp, vp = (a.astype(np.float64) for a in w.kv(0))
            outs[exact, mirror] = od.decode_layer(x, lw, kp, vp, w.page_tables[0], 40, TINY7, exact, mirror)
    assert np.array_equal(outs[True, False], outs[True, True])
    ref = outs[True, False]
    rms = np.sqrt((ref ** 2).mean())
    for mirror in (False, True):   # fp16 rounding of intermediates only: small against the outputs' scale
        assert np.abs(outs[False, mirror] - ref).max() <= 1e-2 * rms
    assert not np.array_equal(outs[False, False], outs[False, True])


# ------------------------------------------------------------------ attention

def _pool_from_logical(k_log, v_log, perm):
    """Scatter logical KV [Hkv, ctx, D] into pages given a physical page list."""
    hkv, ctx, d = k_log.shape
    npg = (ctx + 15) // 16
    kp = np.full((max(perm) + 1, hkv, 16, d), np.nan)
    vp = np.full_like(kp, np.nan)
    for t in range(ctx):
        kp[perm[t // 16], :, t % 16] = k_log[:, t]
        vp[perm[t // 16], :, t % 16] = v_log[:, t]
    return kp, vp


def test_attention_hand_example_d2():
    """Scores 0 and ln 3 -> softmax (1/4, 3/4); V rows (4, 0) and (0, 8) -> o = (1, 6)."""
    q = np.array([[math.sqrt(2) * math.log(3), 0.0]])
    k_log = np.array([[[0.0, 0.0], [1.0, 0.0]]])
    v_log = np.array([[[4.0, 0.0], [0.0, 8.0]]])
    kp, vp = _pool_from_logical(k_log, v_log, [3])
    o = od.attention_decode(q, kp, vp, np.array([3]), 2, exact=True)
    assert np.allclose(o, [[1.0, 6.0]], atol=1e-14)


def test_attention_closed_forms():
    rs = np.random.default_rng(6)
    d, ctx = 128, 37
    q = rs.standard_normal((7, d))
    v_log = rs.standard_normal((1, ctx, d))
    k_log = rs.standard_normal((1, ctx, d))
    perm = [2, 0, 1]
    # ctx = 1 -> o = V_0
    kp, vp = _pool_from_logical(k_log[:, :1], v_log[:, :1], [5])
    assert np.array_equal(od.attention_decode(q, kp, vp, np.array([5]), 1, exact=True),
                          np.repeat(v_log[:, 0], 7, axis=0))
    # V == 1 -> o = 1
    kp, vp = _pool_from_logical(k_log, np.ones_like(v_log), perm)
    assert np.allclose(od.attention_decode(q, kp, vp, np.array(perm), ctx, exact=True), 1.0, atol=1e-14)
    # K constant -> uniform weights -> o = mean(V)
    kp, vp = _pool_from_logical(np.ones_like(k_log) * 0.3, v_log, perm)
    o = od.attention_decode(q, kp, vp, np.array(perm), ctx, exact=True)
    assert np.allclose(o, np.repeat(v_log.mean(axis=1), 7, axis=0), atol=1e-13)
    # softmax rows sum to 1
    p = od.softmax(rs.standard_normal((7, ctx)) * 20)
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-12)


@pytest.mark.parametrize("tstar", [0, 14, 15, 16, 17, 31, 32, 36])
def test_attention_argmax_probe_reads_the_right_slot(tstar):
    """One dominant score selects V[t*] exactly -- catches off-by-one page or
    slot arithmetic ("Building a Custom LLM Inference Runtime on H100", The
    Three Critical Bugs, Bug 1)."""
    rs = np.random.default_rng(7)
    d, ctx = 64, 37
    k_log = np.zeros((1, ctx, d))
    k_log[0, tstar, 0] = 1.0
    q = np.zeros((7, d))
    q[:, 0] = 1e4
    v_log = rs.standard_normal((1, ctx, d)).astype(np.float16).astype(np.float64)
    perm = [4, 1, 3]
    kp, vp = _pool_from_logical(k_log, v_log, perm)
    o = od.attention_decode(q, kp, vp, np.array(perm + [-1]), ctx)
    assert np.array_equal(o, np.repeat(v_log[:, tstar], 7, axis=0))


def test_paged_equals_contiguous_under_any_permutation():
    """Paging is pure addressing ("Building a Custom LLM Inference Runtime on
    H100", The KV Cache and PagedAttention): any physical placement gives
    bit-identical results, equal to a contiguous layout."""
    rs = np.random.default_rng(8)
    hkv, d, ctx = 2, 64, 75
    q = rs.standard_normal((14, d))
    k_log = rs.standard_normal((hkv, ctx, d))
    v_log = rs.standard_normal((hkv, ctx, d))
    ref = None
    for seed in range(4):
        perm = list(np.random.default_rng(seed).permutation(8)[:5]) if seed else [0, 1, 2, 3, 4]
        kp, vp = _pool_from_logical(k_log, v_log, perm)
        o = od.attention_decode(q, kp, vp, np.array(perm), ctx)
        if ref is None:
            ref = o
        assert np.array_equal(o, ref)
    rep = dense.mha(q, np.repeat(k_log, 7, axis=0), np.repeat(v_log, 7, axis=0))
    assert np.allclose(od.attention_decode(q, *_pool_from_logical(k_log, v_log, [0, 1, 2, 3, 4]),
                                           np.arange(5), ctx, exact=True), rep, atol=1e-12)


def test_lse_merge_of_any_split_equals_single_pass():
    rs = np.random.default_rng(9)
    d, ctx = 128, 300
    q = rs.standard_normal(d) * 3
    k = rs.standard_normal((ctx, d))
    v = rs.standard_normal((ctx, d))
    full = od.softmax(k @ q / math.sqrt(d)) @ v
    for bounds in ([0, 300], [0, 16, 300], [0, 1, 2, 299, 300], list(range(0, 300, 16)) + [300],
                   [0, 150, 151, 300]):
        parts = [od.attention_partial(q, k[a:b], v[a:b]) for a, b in zip(bounds[:-1], bounds[1:])]
        assert np.allclose(od.lse_merge(parts), full, atol=1e-12)


# ------------------------------------------------------------------ whole layer

TINY = wl.Shape(hidden=200, n_heads=4, n_kv_heads=2, head_dim=16, ffn=72, vocab=64, n_layers=1)
TINY7 = wl.Shape(hidden=256, n_heads=7, n_kv_heads=1, head_dim=32, ffn=136, vocab=64, n_layers=1)


@pytest.mark.parametrize("shape,ctx,bias", [(TINY, [37], False), (TINY, [16, 5], True),
                                            (TINY7, [33], True), (TINY7, [1], False)])
def test_layer_matches_dense_brute_force(shape, ctx, bias):
    """Paged oracle (exact mode) == dense brute force to 1e-9."""
    w = wl.custom("tiny", 90, shape, ctx, gamma="random")
    lw = w.layer(0, bias=bias)
    x = w.x_in().astype(np.float64)
    kp, vp = (a.astype(np.float64) for a in w.kv(0))
    for b in range(w.batch):
        c = int(w.ctx_lens[b])
        hist_k = np.stack([od.gather_kv(kp, w.page_tables[b], c - 1, j) for j in range(shape.n_kv_heads)])
        hist_v = np.stack([od.gather_kv(vp, w.page_tables[b], c - 1, j) for j in range(shape.n_kv_heads)])
        ref, k_new, v_new = dense.dense_layer(x[b], lw, hist_k, hist_v, c - 1, shape)
        got = od.decode_layer(x[b], lw, kp, vp, w.page_tables[b], c, shape, exact=True)
        assert np.allclose(got, ref, rtol=1e-9, atol=1e-9)
        page, slot = w.page_tables[b][(c - 1) // 16], (c - 1) % 16
        assert np.allclose(kp[page, :, slot], k_new, atol=1e-12)
        assert np.allclose(vp[page, :, slot], v_new, atol=1e-12)


def test_three_step_stateful_run_crossing_a_page():
    """Steps at positions 14, 15, 16: each step reads the K/V the previous one
    wrote; the paged oracle tracks a dense history that grows by appending."""
    shape = TINY
    w = wl.custom("tiny3", 91, shape, [17], gamma="random")
    lw = w.layer(0, bias=True)
    kp, vp = (a.astype(np.float64) for a in w.kv(0))
    pt = w.page_tables[0]
    hk = np.stack([od.gather_kv(kp, pt, 14, j) for j in range(shape.n_kv_heads)])
    hv = np.stack([od.gather_kv(vp, pt, 14, j) for j in range(shape.n_kv_heads)])
    x = w.x_in()[0].astype(np.float64)
    for ctx in (15, 16, 17):
        got = od.decode_layer(x, lw, kp, vp, pt, ctx, shape, exact=True)
        ref, kn, vn = dense.dense_layer(x, lw, hk, hv, ctx - 1, shape)
        assert np.allclose(got, ref, rtol=1e-9, atol=1e-9)
        hk = np.concatenate([hk, kn[:, None]], axis=1)
        hv = np.concatenate([hv, vn[:, None]], axis=1)
        x = got / 8.0


def test_batched_layer_equals_sequences_one_by_one():
    """runs.layer_batch applies the per-row stages to the whole batch at once:
    it must equal decode_layer run for each sequence in turn (exact mode to
    1e-12, and the written page slots), including ragged contexts."""
    from oracle import runs
    w = wl.custom("tinyb", 93, TINY7, [33, 5, 16, 40], gamma="random")
    lw = w.layer(0, bias=True)
    x = w.x_in().astype(np.float64)
    got, kp, vp = runs.layer_batch(w, 0, x, weights=lw, exact=True)
    kp2, vp2 = (a.astype(np.float64) for a in w.kv(0))
    for b in range(w.batch):
        ref = od.decode_layer(x[b], lw, kp2, vp2, w.page_tables[b], int(w.ctx_lens[b]), TINY7, exact=True)
        assert np.allclose(got[b], ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(kp, kp2, rtol=0, atol=1e-12) and np.allclose(vp, vp2, rtol=0, atol=1e-12)
    sub, _, _ = runs.layer_batch(w, 0, x[[3, 1]], weights=lw, exact=True, rows=[3, 1])
    assert np.allclose(sub, got[[3, 1]], rtol=1e-12, atol=1e-12)


def test_layer_outputs_are_fp16_values():
    w = wl.layer_mini()
    x = w.x_in().astype(np.float64)
    from oracle import runs
    out, kp, vp = runs.layer_batch(w, 0, x)
    assert np.array_equal(out.astype(np.float16).astype(np.float64), out)
    assert np.array_equal(kp.astype(np.float16).astype(np.float64), kp)


def _read_golden(path):
    arrays = {}
    for line in open(path):
        if line.startswith("#"):
            continue
        name, n, *vals = line.split()
        arrays[name] = np.array([int(v, 16) for v in vals], dtype=np.uint16).view(np.float16)
        assert arrays[name].size == int(n)
    return arrays


def test_oracle_reproduces_its_stored_layer_output():
    import os
    from oracle import runs
    g = _read_golden(os.path.join(os.path.dirname(__file__), "golden", "layer_mini_oracle.txt"))
    w = wl.layer_mini()
    out, kp, vp = runs.layer_batch(w, 0, w.x_in().astype(np.float64))
    pos = int(w.positions[0])
    page, slot = int(w.page_tables[0][pos // 16]), pos % 16
    assert np.array_equal(out[0].astype(np.float16), g["x_out"])
    assert np.array_equal(kp[page, :, slot].astype(np.float16).ravel(), g["k_slot"])
    assert np.array_equal(vp[page, :, slot].astype(np.float16).ravel(), g["v_slot"])
