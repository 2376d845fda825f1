"""Host-side validation at the boundary: every error reachable from host
inputs is reported before any device work (CPU only: the calls below never
reach a kernel launch)."""
import numpy as np
import pytest

import w4a16_paged_kv_amd as w4

CFG = w4.make_config(448, 7, 1, 64, 1536, 4096, 1)


def _ok_inputs(batch=2, max_pages=4):
    tokens = np.arange(batch, dtype=np.int32)
    ctx = np.array([64, 20][:batch], dtype=np.int32)
    pos = ctx - 1
    pt = np.full((batch, max_pages), -1, dtype=np.int32)
    pt[0, :4] = [3, 0, 2, 1]
    if batch > 1:
        pt[1, :2] = [5, 4]
    return tokens, pos, pt, ctx


def expect(code, *args):
    with pytest.raises(w4.W4Error) as e:
        w4.w4_validate_step(CFG, *args)
    assert e.value.code == code, str(e.value)


def test_valid_inputs_pass():
    w4.w4_validate_step(CFG, 8, 2, 4, *_ok_inputs())


def test_each_error_is_reported():
    t, p, pt, c = _ok_inputs()
    expect(w4.W4_EINVAL, 8, 1, 4, t, p, pt, c)                  # batch > max_batch
    bad = t.copy(); bad[1] = 4096
    expect(w4.W4_ERANGE, 8, 2, 4, bad, p, pt, c)                 # token >= vocab
    bad = c.copy(); bad[0] = 65
    expect(w4.W4_ERANGE, 8, 2, 4, t, p, pt, bad)                 # ctx > 16 * max_pages
    bad = c.copy(); bad[1] = 0
    expect(w4.W4_ERANGE, 8, 2, 4, t, bad - 1, pt, bad)          # empty context
    bad = p.copy(); bad[0] = 62
    expect(w4.W4_ERANGE, 8, 2, 4, t, bad, pt, c)                 # position != ctx - 1
    bad = pt.copy(); bad[1, 1] = 8
    expect(w4.W4_ERANGE, 8, 2, 4, t, p, bad, c)                  # page id >= num_pages
    bad = pt.copy(); bad[1, 1] = -1
    expect(w4.W4_ERANGE, 8, 2, 4, t, p, bad, c)                  # missing page
    bad = pt.copy(); bad[1, 1] = 1
    c2 = c.copy(); c2[1] = 64; p2 = c2 - 1
    bad[1, 2:] = [2, 1]
    bad[1, :2] = [5, 4]
    expect(w4.W4_ERANGE, 8, 2, 4, t, p2, bad, c2)                # same (page, slot) written twice


def test_unused_page_table_entries_are_ignored():
    t, p, pt, c = _ok_inputs()
    pt[1, 2:] = 12345            # beyond ceil(ctx/16): never read
    w4.w4_validate_step(CFG, 8, 2, 4, t, p, pt, c)


def test_bad_configs_have_no_workspace():
    assert w4.w4_workspace_bytes(w4.make_config(448, 7, 1, 96, 1536, 10, 1), 1, 4) == 0    # head_dim
    assert w4.w4_workspace_bytes(w4.make_config(448, 9, 1, 64, 1536, 10, 1), 1, 4) == 0    # group 9
    assert w4.w4_workspace_bytes(w4.make_config(450, 7, 1, 64, 1536, 10, 1), 1, 4) == 0    # hidden % 8
    assert w4.w4_workspace_bytes(CFG, 17, 4) == 0                                          # batch > 16
    assert w4.w4_workspace_bytes(CFG, 1, 4) > 0


def test_model_create_argument_errors_before_device_work():
    import ctypes
    lw = (w4.w4_layer_weights * 1)()
    lw[0] = w4.w4_layer_weights(0x10000, 0x10000, 0x10000, 0x10000, 0x10000, 0x10000, None)
    wts = w4.w4_weights(lw, None, None, None)
    h = ctypes.c_void_p()
    need = w4.w4_workspace_bytes(CFG, 1, 4)
    rc = w4.lib().w4_model_create(ctypes.byref(CFG), ctypes.byref(wts), 0x20000, 8, 0x30000, need - 1, 1, 4,
                                  ctypes.byref(h))
    assert rc == w4.W4_EINVAL and "workspace" in w4.lib().w4_last_error().decode()
    rc = w4.lib().w4_model_create(ctypes.byref(CFG), ctypes.byref(wts), 0x20010, 8, 0x30000, need, 1, 4,
                                  ctypes.byref(h))
    assert rc == w4.W4_EALIGN
    lw[0] = w4.w4_layer_weights(0x10000, None, 0x10000, 0x10000, 0x10000, 0x10000, None)
    rc = w4.lib().w4_model_create(ctypes.byref(CFG), ctypes.byref(wts), 0x20000, 8, 0x30000, need, 1, 4,
                                  ctypes.byref(h))
    assert rc == w4.W4_EINVAL


def test_kernel_entry_argument_errors():
    L = w4.lib()
    assert L.w4_gemv(0x1000, 0x2000, 0x3000, 16, 12, 1, None) == w4.W4_EINVAL          # k % 8
    assert L.w4_gemv(0x1000, 0x2000, 0x3000, 16, 128, 0, None) == w4.W4_EINVAL         # batch
    assert L.w4_gemv(0x1000, 0x2000, 0x3000, 16, 128, (1 << 20) + 1, None) == w4.W4_EINVAL
    assert L.w4_gemv(0x1010, 0x2000, 0x3000, 16, 128, 1, None) == w4.W4_EALIGN
    assert L.w4_gemv_f16(None, 0x2000, 0x3000, 16, 128, 1, None) == w4.W4_EINVAL
    need = L.paged_attention_workspace_bytes(2, 28, 4, 128, 8)
    assert need > 0
    assert L.paged_attention_workspace_bytes(2, 28, 4, 96, 8) == 0
    args = [0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 2, 28, 4, 128, 16, 8, 0x6000]
    assert L.paged_attention_decode(*args, need - 1, 0x7000, None) == w4.W4_EINVAL
    args[1] = 0x2008
    assert L.paged_attention_decode(*args, need, 0x7000, None) == w4.W4_EALIGN


def test_argmax_argument_checks_return_before_device_work():
    """w4_argmax_f16 validates on the host and enqueues nothing on an error
    (the addresses below are never dereferenced)."""
    import ctypes
    import w4a16_paged_kv_amd as w4
    lib = w4.lib()
    assert w4.w4_argmax_workspace_bytes(0, 10) == 0
    assert w4.w4_argmax_workspace_bytes(1, 0) == 0
    assert w4.w4_argmax_workspace_bytes(2, 152064) == 2 * 64 * 8
    assert w4.w4_argmax_workspace_bytes(3, 7) == 3 * 8
    a = 1 << 20                                   # aligned fake addresses
    ok = lib.w4_argmax_f16
    assert ok(None, 1, 10, a, 64, a, None) == w4.W4_EINVAL
    assert ok(a, 0, 10, a, 64, a, None) == w4.W4_EINVAL
    assert ok(a, 1, 0, a, 64, a, None) == w4.W4_EINVAL
    assert ok(a + 2, 1, 10, a, 64, a, None) == w4.W4_EALIGN
    assert ok(a, 1, 10, a + 8, 64, a, None) == w4.W4_EALIGN
    assert ok(a, 2, 152064, a, 2 * 64 * 8 - 1, a, None) == w4.W4_EINVAL
    assert b"workspace" in lib.w4_last_error()


def test_prefill_and_kv_copy_argument_errors():
    """Host checks of the prefill and KV page-copy entry points (no device work)."""
    L = w4.lib()
    cfg = w4.make_config(448, 7, 1, 64, 1536, 5000, 2, 1e-6, 1e6)
    import ctypes
    assert L.w4_prefill_workspace_bytes(ctypes.byref(cfg), 512, 32) > 0
    assert L.w4_prefill_workspace_bytes(ctypes.byref(cfg), 0, 32) == 0
    assert L.w4_prefill(None, None, 1, 0, None, None, 0, None, None) == w4.W4_ESTATE      # no model
    args = (0x1000, 4, 0)   # kv_cache, num_pages, layer
    assert L.kv_write_pages(ctypes.byref(cfg), *args, 0x2000, 2, 20, 13, 0x3000, 0x4000, None) == w4.W4_ERANGE
    assert L.kv_write_pages(ctypes.byref(cfg), *args, 0x2000, 2, 0, 8, 0x3010, 0x4000, None) == w4.W4_EALIGN
    assert L.kv_read_pages(ctypes.byref(cfg), 0x1000, 4, 2, 0x2000, 2, 0, 8, 0x3000, 0x4000, None) == w4.W4_EINVAL
    assert L.kv_read_pages(None, 0x1000, 4, 0, 0x2000, 2, 0, 8, 0x3000, 0x4000, None) == w4.W4_EINVAL

