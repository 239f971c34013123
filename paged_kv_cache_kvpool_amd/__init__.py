"""Paged-KV-pool attention for MI355X (gfx950): decode, speculative verification and
prefix-reuse chunked prefill over a block-paged KV pool.

The compute lives in ``libkvpool.so`` (hand-written HIP kernels behind the C ABI declared in
``include/kvpool.h``).  ``paged_kv_cache_kvpool_amd.binding`` is its ctypes binding (loaded on
first use, importing torch); ``paged_kv_cache_kvpool_amd.workloads`` draws seeded inputs.
"""

_BINDING_NAMES = {
    "kvpool_storage_bytes", "kvpool_scale_bytes", "kvpool_create", "kvpool_create_int8",
    "kvpool_destroy", "kvpool_append",
    "kvpool_copy_blocks", "kvattn_workspace_size", "kvattn_forward", "kvattn_forward_sparse",
    "kvattn_append_forward", "kvattn_append_forward_sparse",
    "kvpool_last_error",
    "kvpool_profile", "kvpool_profile_kernel", "kernel_times",
    "PagedKVPool", "HostStore", "KVPoolError", "KV_F32", "KV_BF16", "KV_I8", "lib",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
