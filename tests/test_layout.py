"""Device V page layout (host side, no GPU): v_pages_device puts value
(token t, dim d) of a (page, head) slice at the element the attention's
P V operands read, and v_pages_host inverts it."""
import numpy as np
import pytest
import torch

from workloads.device import v_pages_device, v_pages_host


def v_offset(t, d):
    # lane d % 16 + 16 (t // 4) holds tokens 4 (t // 4) .. +4 of dims in two
    # neighbouring 16-dim slices: 16 contiguous bytes per lane and slice pair
    lane = d % 16 + 16 * (t // 4)
    return ((d // 32) * 64 + lane) * 8 + ((d // 16) % 2) * 4 + t % 4


@pytest.mark.parametrize("D", [64, 128])
def test_v_pages_device_order(D):
    v = np.arange(16 * D, dtype=np.int32).reshape(16, D)
    flat = v_pages_device(v).reshape(-1)
    offs = np.array([[v_offset(t, d) for d in range(D)] for t in range(16)])
    assert sorted(offs.reshape(-1).tolist()) == list(range(16 * D))   # a permutation
    for t in range(16):
        for d in range(D):
            assert flat[offs[t, d]] == v[t, d]


def test_v_pages_roundtrip_batched():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((3, 2, 4, 16, 128)).astype(np.float16)
    vd = v_pages_device(v)
    assert vd.shape == v.shape
    assert np.array_equal(v_pages_host(vd), v)
    assert torch.equal(v_pages_host(torch.from_numpy(vd)), torch.from_numpy(v))
    # one lane's 16 bytes: tokens 0..3 of dims 0 and 16 (slices 0 and 1)
    assert np.array_equal(vd[1, 1, 2].reshape(-1)[:8], np.concatenate([v[1, 1, 2, :4, 0], v[1, 1, 2, :4, 16]]))
