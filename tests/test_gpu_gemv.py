"""W4A16 GEMV / skinny-GEMM kernels against the oracle (fp64 dequant-matvec)."""
import numpy as np
import pytest
import torch

import w4a16_paged_kv_amd as w4
import workloads as wl
from oracle import decode as od
from tests.gpu_util import assert_close, to_np16
from workloads.device import to_dev

pytestmark = pytest.mark.gpu

SHAPES = [  # (n, k): miniature and Qwen2.5-7B projection shapes, incl. a partial group (k = 448)
    (576, 448), (448, 448), (3072, 448), (448, 1536),
    (4608, 3584), (3584, 3584), (37888, 3584), (3584, 18944), (40, 200),
    # many tiles per workgroup with few groups: batch-1 runs of one or two
    # blocks crossing tiles (6 and 16 tiles per workgroup), and batch > 1
    # shapes past one workgroup per CU
    (24000, 256), (65536, 128)]


@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("batch", [1, 3, 16])
def test_w4_gemv_matches_oracle(n, k, batch):
    if k % 8:
        pytest.skip("activation length must be a multiple of 8")
    print(f"w4_gemv n={n} k={k} batch={batch}", flush=True)
    q, s = wl.int4_matrix(77, 0, 0, n, k)
    x = wl.f16_normal(wl.rng(77, 0, 1), (batch, k))
    packed = to_dev(w4.pack_weights_w4g128(q, s))
    xd = to_dev(x)
    y = torch.empty((batch, n), dtype=torch.float16, device="cuda")
    w4.w4_gemv(packed, xd, y, n, k, batch)
    torch.cuda.synchronize()
    got = to_np16(y)
    for b in range(batch):
        assert_close(got[b], od.r16(od.gemv_w4(q, s, x[b])), f"row {b}")


@pytest.mark.parametrize("n,k", [(600, 448), (1000, 4224), (300, 200)])
@pytest.mark.parametrize("batch", [2, 8, 9, 15])
def test_w4_gemv_batches_across_the_row_halves(n, k, batch):
    """Batch 2..15: the activation rows are staged by two halves of the
    workgroup's threads (rows 0-7 and 8-15), so these batches leave one half
    partly or wholly empty; k = 448 and 200 end inside a group, k = 4224 (33
    groups) needs a second activation window."""
    print(f"w4_gemv n={n} k={k} batch={batch}", flush=True)
    q, s = wl.int4_matrix(79, 0, 0, n, k)
    x = wl.f16_normal(wl.rng(79, 0, 1), (batch, k))
    y = torch.empty((batch, n), dtype=torch.float16, device="cuda")
    w4.w4_gemv(to_dev(w4.pack_weights_w4g128(q, s)), to_dev(x), y, n, k, batch)
    torch.cuda.synchronize()
    got = to_np16(y)
    for b in range(batch):
        assert_close(got[b], od.r16(od.gemv_w4(q, s, x[b])), f"batch {batch} row {b}")


def test_w4_gemv_one_hot_is_exact():
    n, k = 256, 384
    q, s = wl.int4_matrix(78, 0, 0, n, k)
    s[:] = np.float16(1.0)
    x = np.zeros((1, k), np.float16)
    x[0, 131] = 1.0
    y = torch.empty((1, n), dtype=torch.float16, device="cuda")
    w4.w4_gemv(to_dev(w4.pack_weights_w4g128(q, s)), to_dev(x), y, n, k, 1)
    assert np.array_equal(to_np16(y)[0], q[:, 131].astype(np.float16))


@pytest.mark.parametrize("n,k,batch", [(16384, 3584, 1), (4000, 3584, 16), (1000, 448, 5), (152064, 3584, 1),
                                       (152064, 3584, 16), (37, 24, 2), (700, 200, 15), (2000, 4064, 16),
                                       (1500, 4096, 9)])
def test_f16_gemv_matches_oracle(n, k, batch):
    print(f"w4_gemv_f16 n={n} k={k} batch={batch}", flush=True)
    g = wl.rng(79, 0, 0)
    wgt = wl.f16_normal(g, (n, k), 0.02)
    x = wl.f16_normal(g, (batch, k))
    y = torch.empty((batch, n), dtype=torch.float16, device="cuda")
    w4.w4_gemv_f16(to_dev(w4.pack_weights_f16(wgt)), to_dev(x), y, n, k, batch)
    torch.cuda.synchronize()
    got = to_np16(y)
    rows = np.arange(n) if n <= 16384 else np.random.default_rng(0).choice(n, 4096, replace=False)
    ref = od.r16(wgt[rows].astype(np.float64) @ x.astype(np.float64).T).T
    assert_close(got[:, rows], ref, "f16 gemv")


@pytest.mark.parametrize("n,k,batch", [(9, 1000, 16), (300, 1000, 3), (4099, 3584, 16), (40, 24, 7)])
def test_f16_gemm_batched_stays_in_its_outputs_and_repeats(n, k, batch):
    """Batch 2..16 lm_head: every output of the ragged last tile and of
    wavefronts whose second tile lies past the end (their re-read blocks are
    not stored) is written, nothing past the batch x n outputs changes, and a
    second call gives the same bits (one 16 x 16 tile at n = 9; a partial last
    32-column chunk at k = 1000; one chunk at k = 24)."""
    print(f"w4_gemv_f16 guard n={n} k={k} batch={batch}", flush=True)
    g = wl.rng(80, n, k)
    wgt = wl.f16_normal(g, (n, k), 0.02)
    x = wl.f16_normal(g, (batch, k))
    guard = 4096
    ybuf = torch.full((batch * n + guard,), float("nan"), dtype=torch.float16, device="cuda")
    y = ybuf[:batch * n].view(batch, n)
    wd, xd = to_dev(w4.pack_weights_f16(wgt)), to_dev(x)
    w4.w4_gemv_f16(wd, xd, y, n, k, batch)
    torch.cuda.synchronize()
    got = to_np16(y)
    assert not np.isnan(got).any(), "an output was not written"
    assert torch.isnan(ybuf[batch * n:]).all(), "a value past the outputs changed"
    ref = od.r16(wgt.astype(np.float64) @ x.astype(np.float64).T).T
    assert_close(got, ref, "f16 gemm batched")
    w4.w4_gemv_f16(wd, xd, y, n, k, batch)
    torch.cuda.synchronize()
    assert np.array_equal(to_np16(y).view(np.uint16), got.view(np.uint16)), "second call differs"
