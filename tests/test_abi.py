"""The C-ABI library loads and exports every entry point include/kvpool.h declares; host-side
argument checks answer without touching a GPU (CPU only)."""
import ctypes
import os
import re

import pytest

from paged_kv_cache_kvpool_amd import binding as kb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvpool.h")

if not os.path.exists(kb.LIB_PATH):  # pragma: no cover
    pytest.skip("libkvpool.so not built (run __graft_entry__.build())", allow_module_level=True)


def declared():
    text = open(HEADER).read()
    return re.findall(r"KVPOOL_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_header_declares_the_abi():
    names = declared()
    assert set(names) == set(kb.SIGNATURES), names


def test_every_declared_symbol_is_exported():
    lib = kb.lib()
    for name in declared():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_storage_bytes():
    assert kb.kvpool_storage_bytes(2, 10, 16, 8, 128, kb.KV_BF16) == 2 * 10 * 16 * 8 * 128 * 2
    assert kb.kvpool_storage_bytes(1, 3, 64, 1, 64, kb.KV_F32) == 3 * 64 * 64 * 4
    assert kb.kvpool_storage_bytes(2, 10, 16, 8, 128, kb.KV_I8) == 2 * 10 * 16 * 8 * 128
    assert kb.kvpool_scale_bytes(2, 10, 16, 8) == 2 * 10 * 8 * 16 * 4


def test_int8_pool_needs_its_own_create():
    """kvpool_create refuses KV_I8; kvpool_create_int8 refuses missing or misaligned scale arrays
    (host-side checks, no GPU involved)."""
    lib = kb.lib()
    h = ctypes.c_void_p(0)
    assert lib.kvpool_create(ctypes.byref(h), 1, 4, 16, 1, 128, kb.KV_I8, 16, 16) == kb.KV_EINVAL
    assert lib.kvpool_create_int8(ctypes.byref(h), 1, 4, 16, 1, 128, 16, 16, None, 16) == kb.KV_EINVAL
    assert lib.kvpool_create_int8(ctypes.byref(h), 1, 4, 16, 1, 128, 16, 16, 16, 8) == kb.KV_EINVAL
    assert lib.kvpool_create_int8(ctypes.byref(h), 1, 4, 48, 1, 128, 16, 16, 16, 16) == kb.KV_EUNSUPPORTED
    assert h.value is None


@pytest.mark.parametrize("args,code", [
    ((1, 4, 32, 1, 128, kb.KV_BF16), kb.KV_EUNSUPPORTED),   # block size
    ((1, 4, 16, 1, 96, kb.KV_BF16), kb.KV_EUNSUPPORTED),    # head dim
    ((1, 4, 16, 1, 128, 7), kb.KV_EUNSUPPORTED),            # dtype
    ((0, 4, 16, 1, 128, kb.KV_BF16), kb.KV_EINVAL),         # layers
    ((1, 4, 16, 0, 128, kb.KV_BF16), kb.KV_EINVAL),         # kv heads
])
def test_storage_bytes_rejects(args, code):
    with pytest.raises(kb.KVPoolError) as e:
        kb.kvpool_storage_bytes(*args)
    assert e.value.code == code
    assert kb.kvpool_last_error()


def test_create_rejects_before_any_device_call():
    lib = kb.lib()
    assert lib.kvpool_create(None, 1, 4, 16, 1, 128, kb.KV_BF16, 16, 16) == kb.KV_EINVAL
    h = ctypes.c_void_p(0)
    assert lib.kvpool_create(ctypes.byref(h), 1, 4, 16, 1, 128, kb.KV_BF16, None, 16) == kb.KV_EINVAL
    assert lib.kvpool_create(ctypes.byref(h), 1, 4, 16, 1, 128, kb.KV_BF16, 8, 16) == kb.KV_EINVAL
    assert lib.kvpool_create(ctypes.byref(h), 1, 4, 48, 1, 128, kb.KV_BF16, 16, 16) == kb.KV_EUNSUPPORTED
    assert h.value is None


def test_null_handles():
    lib = kb.lib()
    assert lib.kvpool_destroy(None) == kb.KV_OK
    assert lib.kvattn_forward(None, 0, None, None, 8, 1.0, None, 1, None, None, 1, 1, 1, 1,
                              None, None, 0, None) == kb.KV_EINVAL
    assert lib.kvattn_forward_sparse(None, 0, None, None, 8, 1.0, None, 1, None, None, 1, 1, 1, 1,
                                     16, 4096, 16384, None, None, 0, None) == kb.KV_EINVAL
    assert lib.kvpool_append(None, 0, None, None, None, 1, None, None, 1, 1, 1, None) == kb.KV_EINVAL
    assert lib.kvattn_append_forward(None, 0, None, None, None, None, 8, 1.0, None, 1, None, None,
                                     1, 1, 1, 1, None, None, 0, None) == kb.KV_EINVAL
    assert lib.kvattn_append_forward_sparse(None, 0, None, None, None, None, 8, 1.0, None, 1,
                                            None, None, 1, 1, 1, 1, 16, 4096, 16384, None, None,
                                            0, None) == kb.KV_EINVAL
    assert lib.kvpool_copy_blocks(None, None, None, 1, None) == kb.KV_EINVAL
    sz = ctypes.c_size_t(0)
    assert lib.kvattn_workspace_size(None, 8, 1, 1, 1, 1, None, ctypes.byref(sz)) == kb.KV_EINVAL
    assert "NULL" in kb.kvpool_last_error()


@pytest.mark.parametrize("sink,window,min_len", [(-1, 4096, 16384), (16, 0, 16384), (16, 4096, -1)])
def test_sparse_rejects_bad_parameters(sink, window, min_len):
    """The sparse parameters are checked before anything else (no pool, no GPU needed)."""
    lib = kb.lib()
    assert lib.kvattn_forward_sparse(None, 0, None, None, 8, 1.0, None, 1, None, None, 1, 1, 1, 1,
                                     sink, window, min_len, None, None, 0, None) == kb.KV_EINVAL
    assert "sparse" in kb.kvpool_last_error()
    assert lib.kvattn_append_forward_sparse(None, 0, None, None, None, None, 8, 1.0, None, 1,
                                            None, None, 1, 1, 1, 1, sink, window, min_len, None,
                                            None, 0, None) == kb.KV_EINVAL
    assert "sparse" in kb.kvpool_last_error()


def test_host_store_null_arguments():
    """The host page store's entry points refuse NULL handles before any device call."""
    lib = kb.lib()
    h = ctypes.c_void_p(0)
    assert lib.kvhost_create(None, None, 1 << 20) == kb.KV_EINVAL
    assert lib.kvhost_create(ctypes.byref(h), None, 1 << 20) == kb.KV_EINVAL
    assert h.value is None
    assert lib.kvhost_destroy(None) == kb.KV_OK
    assert lib.kvhost_park(None, None, None, 1, None, None) == kb.KV_EINVAL
    assert lib.kvhost_restore(None, None, None, None, 1, None) == kb.KV_EINVAL
    assert lib.kvhost_release(None, None, 1) == kb.KV_EINVAL
    assert lib.kvhost_page_hash(None, None, None, 1, None, None) == kb.KV_EINVAL
    sz = ctypes.c_size_t(0)
    assert lib.kvhost_page_bytes(None, ctypes.byref(sz)) == kb.KV_EINVAL
    a = ctypes.c_int64()
    assert lib.kvhost_stats(None, ctypes.byref(a), ctypes.byref(a), ctypes.byref(a)) == kb.KV_EINVAL
