"""The library's INT4 g128 quantiser (quantize_w4g128, host code) against
the oracle's, bit for bit ("How to build your own LLM runtime from scratch",
"Architectural decisions and optimizations": symmetric group-wise INT4,
group 128)."""
import numpy as np
import pytest

import w4a16_paged_kv_amd as w4
from oracle import quantize as oq


@pytest.mark.parametrize("n,k", [(1, 1), (3, 127), (5, 128), (7, 448), (16, 3584)])
def test_library_quantiser_equals_oracle_bit_exactly(n, k):
    rs = np.random.default_rng(7 + n + k)
    w = (rs.standard_normal((n, k)) * rs.choice([1e-6, 0.02, 3.0, 2000.0])).astype(np.float16)
    w[0, : min(k, 5)] = [0.5, -0.5, 1.5, 2.5, -3.5][: min(k, 5)]   # halfway cases once s = 1 / 2 / ...
    if n > 2:
        w[2] = 0
    q, s = w4.quantize_w4g128(w)
    q0, s0 = oq.quantize_w4g128(w)
    assert np.array_equal(q, q0)
    assert np.array_equal(s.view(np.uint16), s0.view(np.uint16))


def test_library_quantiser_rejects_non_finite_weights():
    w = np.zeros((2, 130), dtype=np.float16)
    w[1, 129] = np.inf
    with pytest.raises(w4.W4Error, match="ERANGE"):
        w4.quantize_w4g128(w)
    w[1, 129] = np.nan
    with pytest.raises(w4.W4Error, match="ERANGE"):
        w4.quantize_w4g128(w)


@pytest.mark.gpu
@pytest.mark.parametrize("n,k,batch", [(576, 448, 1), (4608, 3584, 1), (448, 1536, 16)])
def test_quantised_weights_through_the_gpu_gemv(n, k, batch):
    """fp16 weights -> quantize_w4g128 -> pack_weights_w4g128 -> w4_gemv on the
    GPU, against the oracle's GEMV of the oracle's own quantisation."""
    import torch
    from oracle import decode as od
    from tests.gpu_util import assert_close, to_np16
    from workloads.device import to_dev

    print(f"quantised gemv n={n} k={k} batch={batch}", flush=True)
    rs = np.random.default_rng(n + k)
    wf = (rs.standard_normal((n, k)) * 0.02).astype(np.float16)
    x = rs.standard_normal((batch, k)).astype(np.float16)
    q, s = w4.quantize_w4g128(wf)
    packed = to_dev(w4.pack_weights_w4g128(q, s))
    y = torch.empty((batch, n), dtype=torch.float16, device="cuda")
    w4.w4_gemv(packed, to_dev(x), y, n, k, batch)
    torch.cuda.synchronize()
    q0, s0 = oq.quantize_w4g128(wf)
    got = to_np16(y)
    for b in range(batch):
        assert_close(got[b], od.r16(od.gemv_w4(q0, s0, x[b])), f"row {b}")
