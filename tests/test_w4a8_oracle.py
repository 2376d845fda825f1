"""Pins of the W4A8 variant's oracle (CPU only): the activation quantiser on
hand examples (halves to even, zero rows, negative maxima), the product
reducing exactly to the W4A16 oracle when the activations already lie on the
INT8 grid, exact scaling by powers of two, and the quantisation error bound
("How to build your own LLM runtime from scratch", Architectural decisions
and optimizations: the INT8-activation path the pages measured against the
INT4 unpack)."""
import numpy as np

import workloads as wl
from oracle import decode as od
from oracle import w4a8


def test_quantiser_hand_examples():
    x = np.array([[127.0, -63.5, 0.5, 1.5, 2.5, -0.5]], np.float16)
    xq, s = w4a8.quantize_rows_int8(x)
    assert s.tolist() == [1.0]
    assert xq.tolist() == [[127, -64, 0, 2, 2, 0]]             # halves to even
    xq, s = w4a8.quantize_rows_int8(np.zeros((2, 8), np.float16))
    assert s.tolist() == [0.0, 0.0] and not xq.any()
    xq, s = w4a8.quantize_rows_int8(np.array([[254.0, -2.0, 3.0]], np.float16))
    assert s.tolist() == [2.0] and xq.tolist() == [[127, -1, 2]]  # 3 / 2 = 1.5 -> 2
    xq, s = w4a8.quantize_rows_int8(np.array([[-3.0, 1.0]], np.float16))
    assert s[0] == np.float32(3.0) / np.float32(127.0)
    assert xq.tolist() == [[-127, 42]]                          # 1 / (3/127) = 42.33


def test_on_grid_activations_reduce_to_the_w4a16_oracle():
    rs = np.random.default_rng(0)
    q, s = wl.int4_matrix(60, 0, 0, 40, 448)
    x = rs.integers(-127, 128, (3, 448)).astype(np.float16)
    x[:, 5] = 127.0                                               # max |x| = 127 -> s_x = 1
    assert np.array_equal(w4a8.gemv_w4a8(q, s, x), od.r16(od.gemv_w4(q, s, x)))


def test_power_of_two_scaling_is_exact():
    q, s = wl.int4_matrix(61, 0, 0, 32, 256)
    x = wl.f16_normal(wl.rng(61, 0, 1), (2, 256))
    a = w4a8.gemv_w4a8(q, s, x)
    b = w4a8.gemv_w4a8(q, s, (x.astype(np.float32) * 8).astype(np.float16))
    assert np.array_equal(a * 8, b)


def test_quantisation_error_bound():
    """|W4A8 - W4A16 (exact)| <= s_x / 2 * sum_k |W[n, k]| + fp16 rounding of both."""
    q, s = wl.int4_matrix(62, 0, 0, 64, 384)
    x = wl.f16_normal(wl.rng(62, 0, 1), (4, 384))
    y8 = w4a8.gemv_w4a8(q, s, x)
    y16 = od.gemv_w4(q, s, x)
    _, sx = w4a8.quantize_rows_int8(x)
    wabs = np.abs(od.dequant_w4g128(q, s)).sum(axis=1)
    bound = sx[:, None].astype(np.float64) / 2 * wabs[None, :] + 2 ** -10 * (np.abs(y16) + np.abs(y8))
    assert np.all(np.abs(y8 - y16) <= bound)
    assert np.abs(y8 - y16).max() > 0                            # the variant does differ
