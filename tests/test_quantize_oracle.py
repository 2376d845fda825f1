"""Pins of the oracle's INT4 g128 quantiser ("How to build your own LLM
runtime from scratch", "Architectural decisions and optimizations":
symmetric group-wise INT4, group 128) by closed forms, hand examples and an
exhaustive search over the 16 codes."""
from fractions import Fraction

import numpy as np

from oracle import quantize as oq
from oracle import decode as od


def test_scale_hand_example_and_ties_to_even():
    # max |w| = 7 -> s = 1 exactly; halves go to the even code
    w = np.zeros((1, 128), dtype=np.float16)
    w[0, :6] = [7.0, 2.5, -2.5, 3.5, 0.5, -7.0]
    q, s = oq.quantize_w4g128(w)
    assert s[0, 0] == 1.0
    assert list(q[0, :6]) == [7, 2, -2, 4, 0, -7]
    # max |w| = 1 -> s = fp16(1/7) = 1170 / 8192 (1/7 = 1170.29 / 8192)
    w = np.zeros((1, 128), dtype=np.float16)
    w[0, 3] = -1.0
    q, s = oq.quantize_w4g128(w)
    assert Fraction(float(s[0, 0])) == Fraction(1170, 8192)
    assert q[0, 3] == -7 and (q[0, np.arange(128) != 3] == 0).all()


def test_round_trip_of_exactly_representable_weights():
    """w = q0 * 2^-e with every group holding a +-7: quantisation returns
    (q0, 2^-e) exactly."""
    rs = np.random.default_rng(5)
    n, k = 12, 448
    q0 = rs.integers(-7, 8, (n, k)).astype(np.int8)
    e = rs.integers(3, 12, (n, 4))
    for r in range(n):
        for g in range(4):
            q0[r, 128 * g + rs.integers(0, min(128, k - 128 * g))] = rs.choice([-7, 7])
    s0 = (2.0 ** -e).astype(np.float16)
    w = od.dequant_w4g128(q0, s0).astype(np.float16)
    assert np.array_equal(w.astype(np.float64), od.dequant_w4g128(q0, s0))   # exact in fp16
    q, s = oq.quantize_w4g128(w)
    assert np.array_equal(q, q0) and np.array_equal(s, s0)


def test_codes_minimise_the_error_by_exhaustive_search():
    """Each code is the one of the 16 with the smallest |w - c s| (exact
    rationals), ties to the even code; the scale is the fp16 nearest to
    max|w| / 7; |w - q s| <= s / 2."""
    rs = np.random.default_rng(6)
    w = (rs.standard_normal((6, 300)) * 0.05).astype(np.float16)
    w[2, 128:256] = 0                                          # a zero group
    q, s = oq.quantize_w4g128(w)
    f16 = np.arange(0, 0x7c00, dtype=np.uint16).view(np.float16).astype(np.float64)  # finite non-negative fp16
    for r in range(w.shape[0]):
        for g in range(3):
            lo, hi = 128 * g, min(300, 128 * g + 128)
            m = Fraction(float(np.abs(w[r, lo:hi].astype(np.float64)).max())) / 7
            i = int(np.searchsorted(f16, float(m)))
            nearest = min(abs(Fraction(float(c)) - m) for c in f16[max(0, i - 2): i + 2])
            assert abs(Fraction(float(s[r, g])) - m) == nearest
            sg = Fraction(float(s[r, g]))
            for j in range(lo, hi):
                wj = Fraction(float(w[r, j]))
                if sg == 0:
                    assert q[r, j] == 0
                    continue
                errs = {c: abs(wj - c * sg) for c in range(-8, 8)}
                best = min(errs.values())
                cands = [c for c in errs if errs[c] == best]
                want = cands[0] if len(cands) == 1 else next(c for c in cands if c % 2 == 0)
                assert q[r, j] == want, (r, j)
                assert errs[want] <= sg / 2
    assert (s[2, 1] == 0) and (q[2, 128:256] == 0).all()
