"""KV page pool against a plain Python set model (CPU only)."""
import ctypes

import numpy as np
import pytest

import w4a16_paged_kv_amd as w4


def test_random_alloc_free_matches_set_model():
    rs = np.random.default_rng(0)
    pool = w4.KvPool(200, 4)
    held = []          # list of allocated batches
    free = set(range(200))
    for _ in range(2000):
        if held and rs.random() < 0.45:
            ids = held.pop(rs.integers(len(held)))
            pool.kv_free_pages(ids)
            free |= set(int(i) for i in ids)
        else:
            n = int(rs.integers(0, 12))
            if n > len(free):
                with pytest.raises(w4.W4Error) as e:
                    pool.kv_alloc_pages(n)
                assert e.value.code == w4.W4_ENOPAGES
                assert pool.kv_free_count() == len(free)      # all or nothing
                continue
            ids = pool.kv_alloc_pages(n)
            assert len(set(ids.tolist())) == n and set(ids.tolist()) <= free
            free -= set(ids.tolist())
            held.append(ids)
        assert pool.kv_free_count() == len(free)


def test_double_free_and_range_errors():
    pool = w4.KvPool(8, 1)
    ids = pool.kv_alloc_pages(3)
    pool.kv_free_pages(ids[:1])
    with pytest.raises(w4.W4Error) as e:
        pool.kv_free_pages(ids[:1])
    assert e.value.code == w4.W4_ESTATE
    with pytest.raises(w4.W4Error) as e:
        pool.kv_free_pages([ids[1], ids[1]])
    assert e.value.code == w4.W4_ESTATE
    assert pool.kv_free_count() == 6                      # nothing freed by the failed calls
    with pytest.raises(w4.W4Error) as e:
        pool.kv_free_pages([8])
    assert e.value.code == w4.W4_ERANGE


def test_sequence_growth_and_page_table():
    pool = w4.KvPool(64, 3)
    pool.kv_seq_reserve(0, 16)
    assert pool.kv_seq_pages(0) == 1
    pool.kv_seq_reserve(0, 17)          # crosses a page boundary
    assert pool.kv_seq_pages(0) == 2
    pool.kv_seq_reserve(0, 5)           # never shrinks
    assert pool.kv_seq_pages(0) == 2
    pool.kv_seq_reserve(2, 33)
    pt = pool.page_table([0, 2, 1], 4)
    assert pt.shape == (3, 4)
    assert np.all(pt[0, 2:] == -1) and np.all(pt[1, 3:] == -1) and np.all(pt[2] == -1)
    assert len(set(pt[pt >= 0].tolist())) == 5
    with pytest.raises(w4.W4Error) as e:
        pool.page_table([2], 2)         # holds 3 pages
    assert e.value.code == w4.W4_ERANGE
    owned = pt[0, :2].copy()
    with pytest.raises(w4.W4Error) as e:
        pool.kv_free_pages(owned)       # owned by a sequence
    assert e.value.code == w4.W4_ESTATE
    pool.kv_seq_release(0)
    assert pool.kv_seq_pages(0) == 0 and pool.kv_free_count() == 64 - 3
    with pytest.raises(w4.W4Error):
        pool.kv_seq_reserve(0, 64 * 16)  # exhaustion, all or nothing
    assert pool.kv_seq_pages(0) == 0 and pool.kv_free_count() == 61
    with pytest.raises(w4.W4Error) as e:
        pool.kv_seq_reserve(3, 1)
    assert e.value.code == w4.W4_ERANGE


def test_cache_bytes():
    cfg = w4.make_config(3584, 28, 4, 128, 18944, 152064, 28)
    assert w4.kv_cache_bytes(cfg, 128) == 2 * 28 * 128 * 4 * 16 * 128 * 2


def test_destroyed_pool_is_rejected_and_double_destroy_is_harmless():
    """A destroyed handle is not used: calls report W4_ESTATE (or -1 for the
    counters) instead of reading freed memory, and destroying twice is a
    no-op."""
    lib = w4.lib()
    h = ctypes.c_void_p()
    assert lib.kv_pool_create(16, 2, ctypes.byref(h)) == w4.W4_OK
    lib.kv_pool_destroy(h)
    ids = np.zeros(4, np.int32)
    assert lib.kv_alloc_pages(h, 2, ids.ctypes.data) == w4.W4_ESTATE
    assert lib.kv_free_count(h) == -1
    assert lib.kv_seq_reserve(h, 0, 20) == w4.W4_ESTATE
    assert lib.kv_seq_pages(h, 0) == -1
    lib.kv_pool_destroy(h)
    lib.kv_pool_destroy(None)
