"""The W4A8 variant (INT8 activations on the INT8 matrix cores) and its
same-decomposition W4A16 twin against their oracles (oracle/w4a8.py,
oracle/decode.py); the W4A8 result's distance from the W4A16 oracle is the
accuracy the variant gives up ("How to build your own LLM runtime from
scratch", Architectural decisions and optimizations: the INT8-activation
path the pages dropped)."""
import numpy as np
import pytest
import torch

import w4a16_paged_kv_amd as w4
import workloads as wl
from oracle import decode as od
from oracle import w4a8
from tests.gpu_util import assert_close, to_np16
from workloads.device import to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,k,batch", [(37888, 3584, 1), (37888, 3584, 16), (3584, 18944, 1), (4608, 3584, 4),
                                       (3584, 3584, 1), (576, 448, 3), (40, 200, 2), (448, 1536, 16)])
def test_w4a8_and_w4a16_variants_match_their_oracles(n, k, batch):
    print(f"variant gemv n={n} k={k} batch={batch}", flush=True)
    q, s = wl.int4_matrix(83, 0, 0, n, k)
    x = wl.f16_normal(wl.rng(83, 0, 1), (batch, k))
    x[0, :7] = 0                                     # a few zeros and a tiny row value
    if batch > 1:
        x[1] = 0                                     # a zero row: s_x = 0, y = 0
    packed = to_dev(w4.pack_weights_w4g128(q, s))
    xd = to_dev(x)
    y8 = torch.full((batch, n), float("nan"), dtype=torch.float16, device="cuda")
    y16 = torch.full_like(y8, float("nan"))
    w4.w4_gemv_variant(packed, xd, y8, n, k, batch, int8_activations=True)
    w4.w4_gemv_variant(packed, xd, y16, n, k, batch, int8_activations=False)
    torch.cuda.synchronize()
    ref8 = w4a8.gemv_w4a8(q, s, x)
    ref16 = od.r16(od.gemv_w4(q, s, x))
    assert_close(to_np16(y8), ref8, "W4A8 kernel vs W4A8 oracle")
    assert_close(to_np16(y16), ref16, "W4A16 twin vs W4A16 oracle")
    err = np.abs(ref8 - ref16)
    rel = err / (np.abs(ref16) + 1e-3)
    out = (err > 2e-3 + 1e-2 * np.abs(ref16)).mean()
    print(f"  W4A8 vs W4A16 oracle: {100 * out:.2f}% outside the fp16 tolerance, median relative "
          f"{np.median(rel):.2e}, rms of y {np.sqrt(np.mean(ref16 ** 2)):.3g}", flush=True)


def test_variant_refuses_rows_that_do_not_fit():
    q, s = wl.int4_matrix(84, 0, 0, 16, 18944)
    packed = to_dev(w4.pack_weights_w4g128(q, s))
    x = torch.zeros((16, 18944), dtype=torch.float16, device="cuda")
    y = torch.zeros((16, 16), dtype=torch.float16, device="cuda")
    with pytest.raises(w4.W4Error) as e:
        w4.w4_gemv_variant(packed, x, y, 16, 18944, 16, int8_activations=True)
    assert e.value.code == w4.W4_EINVAL
