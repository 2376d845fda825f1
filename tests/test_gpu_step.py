"""decode_step (embedding, decoder layers, final RMSNorm, fp16 lm_head) against
the oracle; graph replay against eager launches ("Building a Custom LLM
Inference Runtime on H100", CUDA Graph Capture and The Three Critical Bugs,
Bug 3)."""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import runs
from tests.gpu_util import assert_close, to_np16
from tests.staged import full_check
from workloads.device import DeviceModel

pytestmark = pytest.mark.gpu

SMALL = wl.Shape(hidden=448, n_heads=7, n_kv_heads=1, head_dim=64, ffn=1536, vocab=5000, n_layers=3)


def small_model(ctx, gamma="random", wid=30):
    return DeviceModel(wl.custom("small_step", wid, SMALL, ctx, layers=3, lm_head=True, gamma=gamma))


def step(dm, graph=True, inputs=None):
    dm.model.w4_set_graph(graph)
    t, p, pt, c = inputs or dm.step_inputs()
    logits = torch.empty((len(t), dm.w.shape.vocab), dtype=torch.float16, device="cuda")
    dm.model.decode_step(t, p, pt, c, logits)
    torch.cuda.synchronize()
    return to_np16(logits)


@pytest.mark.parametrize("ctx", [[40], [64, 3, 17]])
def test_small_step_matches_oracle(ctx):
    """Every operation of all three layers, the final norm and every lm_head
    row against its oracle stage (GPU inputs fed in), decode_step bit-identical
    to that op-by-op chain and, end to end, within the envelope of the
    oracle's two fp16 placements."""
    full_check(wl.custom("small_step", 30, SMALL, ctx, layers=3, lm_head=True, gamma="random"),
               check_layers={0, 1, 2}, chains=True)


def test_graph_equals_eager_and_replays_are_deterministic():
    dm = small_model([50, 20])
    a = step(dm, graph=False)
    b = step(dm, graph=True)
    c = step(dm, graph=True)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    assert np.array_equal(b.view(np.uint16), c.view(np.uint16))


def test_graph_replays_follow_changing_inputs():
    """One captured graph, new tokens / contexts / page tables every call: each
    of 1000 replays equals an eager run of the same inputs ("Building a Custom
    LLM Inference Runtime on H100", The Three Critical Bugs, Bug 3: inputs
    are staged before the launch, never inside the captured graph)."""
    dm = small_model([60, 30])
    w, m = dm.w, dm.model
    rs = np.random.default_rng(3)
    out_g = torch.empty((2, SMALL.vocab), dtype=torch.float16, device="cuda")   # one output: one graph
    out_e = torch.empty_like(out_g)
    snap = torch.empty_like(dm.kv_cache)
    for it in range(1000):
        c0 = int(rs.integers(1, 16 * w.max_pages + 1))
        room = min(w.max_pages, w.num_pages - (c0 + 15) // 16)     # pages left for the second sequence
        ctx = np.array([c0, rs.integers(1, 16 * room + 1)], np.int32)
        pt = np.full_like(w.page_tables, -1)
        perm = rs.permutation(w.num_pages).astype(np.int32)
        n0, n1 = (ctx + 15) // 16
        pt[0, :n0] = perm[:n0]
        pt[1, :n1] = perm[n0:n0 + n1]
        toks = rs.integers(0, SMALL.vocab, 2).astype(np.int32)
        snap.copy_(dm.kv_cache)
        m.w4_set_graph(True)
        m.decode_step(toks, ctx - 1, pt, ctx, out_g)
        dm.kv_cache.copy_(snap)
        m.w4_set_graph(False)
        m.decode_step(toks, ctx - 1, pt, ctx, out_e)
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), out_e.view(torch.int16)), f"replay {it}"
    assert m.w4_device_errors() == 0


def test_device_inputs_match_host_inputs():
    dm = small_model([45, 9])
    t, p, pt, c = dm.step_inputs()
    a = step(dm, graph=True)
    dev = [torch.from_numpy(np.ascontiguousarray(x, np.int32)).cuda() for x in (t, p, pt, c)]
    logits = torch.empty((2, SMALL.vocab), dtype=torch.float16, device="cuda")
    dm.model.decode_step_device(*dev, logits)
    torch.cuda.synchronize()
    assert np.array_equal(a.view(np.uint16), to_np16(logits).view(np.uint16))
    assert dm.model.w4_device_errors() == 0


@pytest.mark.parametrize("graph", [True, False])
def test_back_to_back_host_input_steps(graph):
    """Six host-input steps enqueued without a synchronisation in between,
    each with its own tokens, positions, page table and context lengths: the
    host staging images are reused while earlier copies may still be queued,
    so every step must still see its own inputs. Reference: the same six steps
    with device-resident inputs from the same initial KV cache (same kernels,
    so bit-identical)."""
    dm = small_model([60, 30])
    w, m = dm.w, dm.model
    rs = np.random.default_rng(11)
    calls = []
    for _ in range(6):
        c0 = int(rs.integers(1, 16 * w.max_pages + 1))
        room = min(w.max_pages, w.num_pages - (c0 + 15) // 16)
        ctx = np.array([c0, rs.integers(1, 16 * room + 1)], np.int32)
        pt = np.full_like(w.page_tables, -1)
        perm = rs.permutation(w.num_pages).astype(np.int32)
        n0, n1 = (ctx + 15) // 16
        pt[0, :n0] = perm[:n0]
        pt[1, :n1] = perm[n0:n0 + n1]
        toks = rs.integers(0, SMALL.vocab, 2).astype(np.int32)
        calls.append((toks, ctx - 1, pt, ctx))
    snap = dm.kv_cache.clone()
    m.w4_set_graph(graph)
    outs = [torch.empty((2, SMALL.vocab), dtype=torch.float16, device="cuda") for _ in calls]
    for (t, p, pt, c), o in zip(calls, outs):
        m.decode_step(t, p, pt, c, o)            # host arrays, no wait between the calls
    torch.cuda.synchronize()
    got = [to_np16(o) for o in outs]
    dm.kv_cache.copy_(snap)
    for i, (t, p, pt, c) in enumerate(calls):
        dev = [torch.from_numpy(np.ascontiguousarray(x, np.int32)).cuda() for x in (t, p, pt, c)]
        ref = torch.empty((2, SMALL.vocab), dtype=torch.float16, device="cuda")
        m.decode_step_device(*dev, ref)
        torch.cuda.synchronize()
        assert np.array_equal(got[i].view(np.uint16), to_np16(ref).view(np.uint16)), f"call {i}"
    assert m.w4_device_errors() == 0


def test_destroy_right_after_an_asynchronous_host_input_step():
    """A model destroyed while its last host-input steps may still be queued
    (no synchronisation in between) releases its staging buffers only after
    their copies ran: the queued steps finish with the inputs they were given."""
    import w4a16_paged_kv_amd as w4
    dm = small_model([45, 9])
    ref = step(dm, graph=True)
    t, p, pt, c = dm.step_inputs()
    outs = [torch.empty((2, SMALL.vocab), dtype=torch.float16, device="cuda") for _ in range(3)]
    snap = dm.kv_cache.clone()
    for o in outs:
        dm.kv_cache.copy_(snap)                  # same KV state for every call (stream-ordered)
        dm.model.decode_step(t, p, pt, c, o)
    h = dm.model.handle
    w4.lib().w4_model_destroy(h)
    dm.model.handle = None
    torch.cuda.synchronize()
    for o in outs:
        assert np.array_equal(to_np16(o).view(np.uint16), ref.view(np.uint16))


def test_destroyed_model_handle_is_rejected():
    """A destroyed model is refused (W4_ESTATE, -1 for the error count), and a
    second destroy does nothing."""
    import w4a16_paged_kv_amd as w4
    dm = small_model([10])
    h = dm.model.handle
    lib = w4.lib()
    lib.w4_model_destroy(h)
    dm.model.handle = None
    assert lib.w4_set_graph(h, 1) == w4.W4_ESTATE
    assert lib.w4_device_errors(h, None) == -1
    assert lib.w4_model_buffer(h, w4.BUF_X, None) is None
    lib.w4_model_destroy(h)
