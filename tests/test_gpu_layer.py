"""decode_layer (one decoder layer: fused qkv/RoPE/KV-write, paged attention,
o-proj + residual, gate/up SiLU-mul, down + residual) against the oracle.

Two kinds of check: operation by operation with the GPU's own inputs fed to
each oracle stage (tests/staged.py; isolates each kernel), and the whole
layer end to end: element by element where the result is insensitive
enough, else within the envelope of the oracle's two fp16 placements.
"""
import os

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import runs
from tests.gpu_util import assert_close, to_np16
from tests.staged import check_envelope, staged_layer
from workloads.device import DeviceModel, k_pages_host, to_dev, v_pages_host

pytestmark = pytest.mark.gpu


def run_layer(dm: DeviceModel, x_in: np.ndarray, layer: int = 0):
    w = dm.w
    xd = to_dev(x_in)
    out = torch.empty_like(xd)
    dm.model.decode_layer(layer, xd, out, w.positions, w.page_tables, w.ctx_lens)
    torch.cuda.synchronize()
    return to_np16(out)


def check_kv_writes_only_the_slot(dm, w, cache0):
    diff = dm.kv_cache.cpu().view(torch.int16) != cache0.cpu().view(torch.int16)    # [L,2,P,Hkv,16,D]
    k_changed = k_pages_host(diff[:, 0]).any(dim=-1)                                  # K slices, device order
    v_changed = v_pages_host(diff[:, 1]).any(dim=-1)                                  # V slices, device order
    changed = torch.stack([k_changed, v_changed], dim=1)                                # [L,2,P,Hkv,16]
    expect = torch.zeros_like(changed)
    for b in range(w.batch):
        pos = int(w.positions[b])
        expect[0, :, int(w.page_tables[b, pos // 16]), :, pos % 16] = True
    assert torch.equal(changed | expect, expect), "a K/V element outside the token's slot changed"
    assert torch.equal(changed, expect), "the token's K/V slot was not written"


def staged(w, bias=False):
    dm = DeviceModel(w, bias=bias)
    cache0 = dm.kv_cache.clone()
    lw = w.layer(0, bias=bias)
    kp, vp = (a.astype(np.float64) for a in w.kv(0))
    staged_layer(dm, w, 0, w.x_in(), lw, kp, vp, w.name)
    check_kv_writes_only_the_slot(dm, w, cache0)
    return dm


def test_layer_mini_end_to_end_and_golden():
    w = wl.layer_mini()
    dm = DeviceModel(w)
    cache0 = dm.kv_cache.clone()
    got = run_layer(dm, w.x_in())
    ref, _, _ = runs.layer_batch(w, 0, w.x_in().astype(np.float64))
    assert_close(got, ref, "layer_mini x_out")
    check_kv_writes_only_the_slot(dm, w, cache0)
    from tests.test_oracle_pins import _read_golden
    g = _read_golden(os.path.join(os.path.dirname(__file__), "golden", "layer_mini_oracle.txt"))
    assert_close(got[0], g["x_out"].astype(np.float64), "golden x_out")


def test_layer_mini_staged():
    staged(wl.layer_mini())


def test_layer_mini_random_gamma_and_bias():
    staged(wl.custom("mini_gb", 20, wl.MINI, [64], gamma="random"), bias=True)


def test_layer_full_shape_staged():
    staged(wl.layer_full())


def test_layer_full_shape_end_to_end_envelope():
    """Whole layer against the oracle's own chain. A 1-ulp difference in an
    intermediate fp16 rounding can reach an output that cancels to near
    zero, so the GPU is held to the envelope of two faithful placements:
    it may disagree with the oracle no more than the oracle's mirror
    placement does (share outside the tolerance and largest error)."""
    w = wl.layer_full()
    dm = DeviceModel(w)
    got = run_layer(dm, w.x_in())
    x = w.x_in().astype(np.float64)
    ref, _, _ = runs.layer_batch(w, 0, x)
    mir, _, _ = runs.layer_batch(w, 0, x, mirror=True)
    check_envelope(got, ref, mir, "layer_full x_out")


@pytest.mark.parametrize("ctx", [[1], [17], [33, 64, 7], [100, 1, 48, 200, 16, 31, 2, 90]])
def test_layer_mini_batches_and_ragged(ctx):
    """Batch 1 uses the VALU GEMVs, batch > 1 the MFMA skinny GEMMs."""
    staged(wl.custom("mini_b", 21, wl.MINI, ctx, gamma="random"), bias=len(ctx) > 2)


def test_layer_full_shape_batch16():
    ctx = wl.rng(22, 0, wl.CTX).integers(1, 700, 16)
    staged(wl.custom("full_b16", 22, wl.QWEN7B, ctx))


@pytest.mark.parametrize("ffn,ctx", [(4480, [40, 3, 129, 77, 16]), (12160, [5, 300, 64])])
def test_layer_long_ffn_split_k(ffn, ctx):
    """Batch > 1 with the down projection's rows longer than one activation
    window (35 and 95 groups): K split over 2 and 3 workgroups per tile group
    (uneven chunks) and the last arrival's sum. The Qwen2.5-7B batch-16 tests
    cover five chunks and a partial last tile group."""
    sh = wl.Shape(hidden=448, n_heads=7, n_kv_heads=1, head_dim=64, ffn=ffn, vocab=64, n_layers=1)
    staged(wl.custom(f"ffn{ffn}", 24, sh, ctx, gamma="random"))


def test_layer_wide_hidden_two_windows():
    """Batch > 1 with hidden 4608 (36 groups, more than one 32-group activation
    window): the RMSNorm'd projections take their sums of squares from a
    pre-pass over the rows and stage them in two windows, the second with 4
    groups of 32."""
    sh = wl.Shape(hidden=4608, n_heads=72, n_kv_heads=9, head_dim=64, ffn=512, vocab=64, n_layers=1)
    staged(wl.custom("wide", 25, sh, [40, 3, 129], gamma="random"), bias=True)

