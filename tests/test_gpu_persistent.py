"""The persistent layer kernel (one launch per decoder layer, its five
operations meeting at grid barriers) runs the per-operation kernels' device
code with the same work split: its logits and K/V writes must equal theirs
bit for bit, over repeated launches (the barrier epochs advance per launch),
and interleaved with the per-operation path (shared attention counters)."""
import numpy as np
import pytest
import torch

import workloads as wl
from tests.gpu_util import to_np16
from workloads.device import DeviceModel

pytestmark = pytest.mark.gpu

SMALL = wl.Shape(hidden=448, n_heads=7, n_kv_heads=1, head_dim=64, ffn=1536, vocab=5000, n_layers=3)


def step(dm, persistent):
    m = dm.model
    m.w4_set_graph(not persistent)
    m.w4_set_persistent(persistent)
    t, p, pt, c = dm.step_inputs()
    logits = torch.empty((len(t), dm.w.shape.vocab), dtype=torch.float16, device="cuda")
    m.decode_step(t, p, pt, c, logits)
    torch.cuda.synchronize()
    return to_np16(logits).view(np.uint16)


@pytest.mark.parametrize("which", ["small", "step_b1"])
def test_persistent_layers_bit_identical(which):
    w = (wl.custom("small_step", 30, SMALL, [40], layers=3, lm_head=True, gamma="random") if which == "small"
         else wl.step_b1())
    dm = DeviceModel(w)
    cache0 = dm.kv_cache.clone()
    ref = step(dm, False)
    kv_ref = dm.kv_cache.clone()
    for i in range(3):
        dm.kv_cache.copy_(cache0)
        got = step(dm, True)
        assert np.array_equal(got, ref), f"launch {i}: logits differ"
        assert torch.equal(dm.kv_cache.view(torch.int16), kv_ref.view(torch.int16)), f"launch {i}: K/V differ"
        assert np.array_equal(step(dm, False), ref), f"launch {i}: per-operation path after the persistent one"
    assert dm.model.w4_device_errors() == 0
