"""The C-ABI library loads and exports every function include/w4a16.h declares (CPU only)."""
import os
import re

import pytest

import w4a16_paged_kv_amd as w4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "w4a16.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*([a-z][a-z0-9_]*)\s*\(", src, re.M))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("pack_weights_w4g128", "kv_alloc_pages", "page_table", "decode_step", "decode_layer",
                 "paged_attention_decode", "w4_model_create", "w4_set_graph"):
        assert must in names
    assert len(names) >= 28


def test_library_exports_every_declared_symbol():
    lib = w4.lib()
    names = declared_functions()
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(names) == sorted(w4.EXPORTED), set(names) ^ set(w4.EXPORTED)


def test_version_and_error_string():
    assert "gfx950" in w4.w4_version()
    with pytest.raises(w4.W4Error) as e:
        w4.KvPool(0, 1)
    assert e.value.code == w4.W4_EINVAL
    assert "num_pages" in str(e.value)
