"""Helpers shared by the GPU tests (tolerance check, host<->device copies)."""
import numpy as np

ATOL, RTOL = 2e-3, 1e-2   # |gpu - oracle| <= 2e-3 + 1e-2 |oracle| on fp16 outputs
F16_MAX = 65504.0


def to_np16(t) -> np.ndarray:
    return t.detach().cpu().contiguous().view(dtype=__import__("torch").int16).numpy().view(np.float16)


def assert_close(gpu, ref, what="", atol=ATOL, rtol=RTOL, max_bad=0):
    """Element-wise |gpu - ref| <= atol + rtol |ref|. Where the oracle's value
    overflows fp16 (it is +-inf after rounding, or within one ulp of the
    largest finite value) the GPU value must be the same infinity or a finite
    value within tolerance; non-finite GPU values are accepted nowhere else."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert not np.isnan(r).any(), f"{what}: NaN in the oracle (compare only finite inputs)"
    edge = np.abs(r) >= F16_MAX - 16.0                      # rounds to inf or to +-65504
    both_inf = np.isinf(g) & edge & (np.sign(g) == np.sign(r))
    if not np.all(np.isfinite(g) | both_inf):
        i = np.argwhere(~(np.isfinite(g) | both_inf))[0]
        raise AssertionError(f"{what}: non-finite GPU value at {tuple(i)}: gpu={g[tuple(i)]!r} oracle={r[tuple(i)]!r}")
    rr = np.where(np.isinf(r), np.sign(r) * F16_MAX, r)
    gg = np.where(both_inf, rr, g)
    err = np.abs(gg - rr)
    bad = err > atol + rtol * np.abs(rr)
    if bad.sum() > max_bad:
        i = np.unravel_index(np.argmax(err - (atol + rtol * np.abs(rr))), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; worst at {i}: "
                             f"gpu={g[i]!r} oracle={r[i]!r} (max abs err {err.max():.3g})")
    return float(err.max())
