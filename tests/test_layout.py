"""Device K and V page layouts (host side, no GPU): k_pages_device and
v_pages_device put value (token t, dim d) of a (page, head) slice at the
element the attention's score and P V operands read, and k_pages_host /
v_pages_host invert them."""
import numpy as np
import pytest
import torch

from workloads.device import k_pages_device, k_pages_host, v_pages_device, v_pages_host


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


def k_offset(t, d):
    # lane t + 16 (chunk of 8 dims within the 32-dim step) holds dims
    # 32 (d // 32) + 8 c .. +8 of token t; a step's 64 lanes are contiguous
    lane = t + 16 * ((d // 8) % 4)
    return ((d // 32) * 64 + lane) * 8 + d % 8


@pytest.mark.parametrize("D", [64, 128])
def test_k_pages_device_order(D):
    k = np.arange(16 * D, dtype=np.int32).reshape(16, D)
    flat = k_pages_device(k).reshape(-1)
    offs = np.array([[k_offset(t, d) for d in range(D)] for t in range(16)])
    assert sorted(offs.reshape(-1).tolist()) == list(range(16 * D))   # a permutation
    for t in range(16):
        for d in range(D):
            assert flat[offs[t, d]] == k[t, d]


def test_k_pages_roundtrip_batched():
    rng = np.random.default_rng(4)
    k = rng.standard_normal((3, 2, 4, 16, 128)).astype(np.float16)
    kd = k_pages_device(k)
    assert kd.shape == k.shape
    assert np.array_equal(k_pages_host(kd), k)
    assert torch.equal(k_pages_host(torch.from_numpy(kd)), torch.from_numpy(k))
    # lane 17's 16 bytes of step 0: token 1, dims 8 .. 16
    assert np.array_equal(kd[0, 1, 3].reshape(-1)[17 * 8:18 * 8], k[0, 1, 3, 1, 8:16])
