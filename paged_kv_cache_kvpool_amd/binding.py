"""ctypes binding of libkvpool.so: one Python function per C entry point, same names.

Argument marshalling only: torch tensors supply device pointers (``data_ptr()``) and the HIP
stream defaults to torch's current stream.  Every step of the computation runs in the
library's HIP kernels; there is no other code path.  If the library is not built, loading
fails with an error (build it with ``python -m paged_kv_cache_kvpool_amd.build``).

torch is imported before the library is loaded so that both use the same HIP runtime
(libamdhip64.so.7 is resolved to the copy torch already loaded).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import numpy as np
import torch

# KVPOOL_LIB: load a library built elsewhere (e.g. another build of the same sources).
LIB_PATH = os.environ.get("KVPOOL_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                        "libkvpool.so")

KV_OK, KV_EINVAL, KV_ERANGE, KV_EUNSUPPORTED, KV_EDEVICE, KV_ENOMEM = 0, -1, -2, -3, -4, -5
KV_F32, KV_BF16, KV_I8 = 0, 1, 2
STATUS_NAMES = {0: "KV_OK", -1: "KV_EINVAL", -2: "KV_ERANGE", -3: "KV_EUNSUPPORTED",
                -4: "KV_EDEVICE", -5: "KV_ENOMEM"}

_i32, _f32, _sz, _vp = ctypes.c_int32, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p

# name -> (restype, argtypes); mirrors include/kvpool.h
SIGNATURES = {
    "kvpool_storage_bytes": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_sz)]),
    "kvpool_create": (_i32, [ctypes.POINTER(_vp), _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp]),
    "kvpool_scale_bytes": (_i32, [_i32, _i32, _i32, _i32, ctypes.POINTER(_sz)]),
    "kvpool_create_int8": (_i32, [ctypes.POINTER(_vp), _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "kvpool_destroy": (_i32, [_vp]),
    "kvpool_append": (_i32, [_vp, _i32, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _vp]),
    "kvpool_copy_blocks": (_i32, [_vp, _vp, _vp, _i32, _vp]),
    "kvattn_workspace_size": (_i32, [_vp, _i32, _i32, _i32, _i32, _i32, _vp, ctypes.POINTER(_sz)]),
    "kvattn_forward": (_i32, [_vp, _i32, _vp, _vp, _i32, _f32, _vp, _i32, _vp, _vp, _i32, _i32,
                              _i32, _i32, _vp, _vp, _sz, _vp]),
    "kvattn_forward_noalloc": (_i32, [_vp, _i32, _vp, _vp, _i32, _f32, _vp, _i32, _vp, _vp, _i32,
                                      _i32, _i32, _i32, _vp, _vp]),
    "kvattn_append_forward": (_i32, [_vp, _i32, _vp, _vp, _vp, _vp, _i32, _f32, _vp, _i32, _vp,
                                     _vp, _i32, _i32, _i32, _i32, _vp, _vp, _sz, _vp]),
    "kvattn_forward_sparse": (_i32, [_vp, _i32, _vp, _vp, _i32, _f32, _vp, _i32, _vp, _vp, _i32,
                                     _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _sz, _vp]),
    "kvattn_append_forward_sparse": (_i32, [_vp, _i32, _vp, _vp, _vp, _vp, _i32, _f32, _vp, _i32,
                                            _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                            _vp, _vp, _sz, _vp]),
    "kvhost_page_bytes": (_i32, [_vp, ctypes.POINTER(_sz)]),
    "kvhost_create": (_i32, [ctypes.POINTER(_vp), _vp, _sz]),
    "kvhost_destroy": (_i32, [_vp]),
    "kvhost_park": (_i32, [_vp, _vp, _vp, _i32, _vp, _vp]),
    "kvhost_restore": (_i32, [_vp, _vp, _vp, _vp, _i32, _vp]),
    "kvhost_release": (_i32, [_vp, _vp, _i32]),
    "kvhost_stats": (_i32, [_vp, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                            ctypes.POINTER(ctypes.c_int64)]),
    "kvhost_page_hash": (_i32, [_vp, _vp, _vp, _i32, _vp, _vp]),
    "kvpool_last_error": (ctypes.c_char_p, []),
    "kvpool_profile": (_i32, [_i32]),
    "kvpool_profile_kernel": (_i32, [_i32, ctypes.POINTER(ctypes.c_char_p),
                                     ctypes.POINTER(_i32), ctypes.POINTER(ctypes.c_double)]),
}


class KVPoolError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {message}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m paged_kv_cache_kvpool_amd.build`")
        cdll = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(cdll, name)
            fn.restype, fn.argtypes = res, args
        _lib = cdll
    return _lib


def _check(rc: int) -> None:
    if rc != KV_OK:
        raise KVPoolError(rc, kvpool_last_error())


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.data_ptr()
    return int(x)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def kvpool_last_error() -> str:
    return lib().kvpool_last_error().decode()


def kvpool_profile(enable: bool) -> None:
    _check(lib().kvpool_profile(1 if enable else 0))


def kvpool_profile_kernel(index: int):
    """(name, launches, total_ms) for one kernel, or None past the last kernel index."""
    name, n, ms = ctypes.c_char_p(), _i32(0), ctypes.c_double(0.0)
    rc = lib().kvpool_profile_kernel(index, ctypes.byref(name), ctypes.byref(n), ctypes.byref(ms))
    if rc == KV_ERANGE:
        return None
    _check(rc)
    return name.value.decode(), n.value, ms.value


def kernel_times() -> dict:
    """{kernel name: (launches, total_ms)} for every kernel launched since kvpool_profile(True)."""
    out, i = {}, 0
    while True:
        r = kvpool_profile_kernel(i)
        if r is None:
            return out
        if r[1]:
            out[r[0]] = (r[1], r[2])
        i += 1


def kvpool_storage_bytes(num_layers, num_blocks, block_size, num_kv_heads, head_dim, dtype) -> int:
    out = _sz(0)
    _check(lib().kvpool_storage_bytes(num_layers, num_blocks, block_size, num_kv_heads, head_dim,
                                      dtype, ctypes.byref(out)))
    return out.value


def kvpool_create(num_layers, num_blocks, block_size, num_kv_heads, head_dim, dtype, k_storage,
                  v_storage) -> int:
    h = _vp(0)
    _check(lib().kvpool_create(ctypes.byref(h), num_layers, num_blocks, block_size, num_kv_heads,
                               head_dim, dtype, _ptr(k_storage), _ptr(v_storage)))
    return h.value


def kvpool_scale_bytes(num_layers, num_blocks, block_size, num_kv_heads) -> int:
    out = _sz(0)
    _check(lib().kvpool_scale_bytes(num_layers, num_blocks, block_size, num_kv_heads,
                                    ctypes.byref(out)))
    return out.value


def kvpool_create_int8(num_layers, num_blocks, block_size, num_kv_heads, head_dim, k_storage,
                       v_storage, k_scales, v_scales) -> int:
    h = _vp(0)
    _check(lib().kvpool_create_int8(ctypes.byref(h), num_layers, num_blocks, block_size,
                                    num_kv_heads, head_dim, _ptr(k_storage), _ptr(v_storage),
                                    _ptr(k_scales), _ptr(v_scales)))
    return h.value


def kvpool_destroy(handle) -> None:
    _check(lib().kvpool_destroy(handle))


def kvpool_append(handle, layer, k_new, v_new, block_tables, max_blocks_per_seq, ctx_lens,
                  q_lens, num_seqs, total_q, max_q_len, stream=None) -> None:
    _check(lib().kvpool_append(handle, layer, _ptr(k_new), _ptr(v_new), _ptr(block_tables),
                               max_blocks_per_seq, _ptr(ctx_lens), _ptr(q_lens), num_seqs,
                               total_q, max_q_len, _stream(stream)))


def kvpool_copy_blocks(handle, src, dst, n, stream=None) -> None:
    _check(lib().kvpool_copy_blocks(handle, _ptr(src), _ptr(dst), n, _stream(stream)))


def _host_i32(x):
    """Host int32 array (kept alive by the caller) and its address, for the q_lens mirror."""
    if x is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(x, dtype=np.int32))
    return arr, arr.ctypes.data


def kvattn_workspace_size(handle, num_q_heads, num_seqs, total_q, max_ctx_len, max_q_len,
                          q_lens_host=None) -> int:
    out = _sz(0)
    arr, addr = _host_i32(q_lens_host)
    _check(lib().kvattn_workspace_size(handle, num_q_heads, num_seqs, total_q, max_ctx_len,
                                       max_q_len, addr, ctypes.byref(out)))
    del arr
    return out.value


def kvattn_forward(handle, layer, q, out, num_q_heads, scale, block_tables, max_blocks_per_seq,
                   ctx_lens, q_lens, num_seqs, total_q, max_ctx_len, max_q_len, workspace,
                   workspace_bytes, stream=None, q_lens_host=None) -> None:
    arr, addr = _host_i32(q_lens_host)
    _check(lib().kvattn_forward(handle, layer, _ptr(q), _ptr(out), num_q_heads, float(scale),
                                _ptr(block_tables), max_blocks_per_seq, _ptr(ctx_lens),
                                _ptr(q_lens), num_seqs, total_q, max_ctx_len, max_q_len, addr,
                                _ptr(workspace), workspace_bytes, _stream(stream)))
    del arr


def kvattn_forward_noalloc(handle, layer, q, out, num_q_heads, scale, block_tables,
                           max_blocks_per_seq, ctx_lens, q_lens, num_seqs, total_q, max_ctx_len,
                           max_q_len, stream=None, q_lens_host=None) -> None:
    """kvattn_forward on the library's static per-GPU scratch (no workspace, no allocation)."""
    arr, addr = _host_i32(q_lens_host)
    _check(lib().kvattn_forward_noalloc(handle, layer, _ptr(q), _ptr(out), num_q_heads,
                                        float(scale), _ptr(block_tables), max_blocks_per_seq,
                                        _ptr(ctx_lens), _ptr(q_lens), num_seqs, total_q,
                                        max_ctx_len, max_q_len, addr, _stream(stream)))
    del arr


KVATTN_NOALLOC_SCRATCH_BYTES = 64 << 20  # include/kvpool.h


def kvattn_append_forward(handle, layer, k_new, v_new, q, out, num_q_heads, scale, block_tables,
                          max_blocks_per_seq, ctx_lens, q_lens, num_seqs, total_q, max_ctx_len,
                          max_q_len, workspace, workspace_bytes, stream=None,
                          q_lens_host=None) -> None:
    arr, addr = _host_i32(q_lens_host)
    _check(lib().kvattn_append_forward(handle, layer, _ptr(k_new), _ptr(v_new), _ptr(q),
                                       _ptr(out), num_q_heads, float(scale), _ptr(block_tables),
                                       max_blocks_per_seq, _ptr(ctx_lens), _ptr(q_lens), num_seqs,
                                       total_q, max_ctx_len, max_q_len, addr, _ptr(workspace),
                                       workspace_bytes, _stream(stream)))
    del arr


def kvattn_forward_sparse(handle, layer, q, out, num_q_heads, scale, block_tables,
                          max_blocks_per_seq, ctx_lens, q_lens, num_seqs, total_q, max_ctx_len,
                          max_q_len, sink_tokens, window_tokens, min_ctx_len, workspace,
                          workspace_bytes, stream=None, q_lens_host=None) -> None:
    arr, addr = _host_i32(q_lens_host)
    _check(lib().kvattn_forward_sparse(handle, layer, _ptr(q), _ptr(out), num_q_heads,
                                       float(scale), _ptr(block_tables), max_blocks_per_seq,
                                       _ptr(ctx_lens), _ptr(q_lens), num_seqs, total_q,
                                       max_ctx_len, max_q_len, sink_tokens, window_tokens,
                                       min_ctx_len, addr, _ptr(workspace), workspace_bytes,
                                       _stream(stream)))
    del arr


def kvattn_append_forward_sparse(handle, layer, k_new, v_new, q, out, num_q_heads, scale,
                                 block_tables, max_blocks_per_seq, ctx_lens, q_lens, num_seqs,
                                 total_q, max_ctx_len, max_q_len, sink_tokens, window_tokens,
                                 min_ctx_len, workspace, workspace_bytes, stream=None,
                                 q_lens_host=None) -> None:
    arr, addr = _host_i32(q_lens_host)
    _check(lib().kvattn_append_forward_sparse(
        handle, layer, _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(out), num_q_heads, float(scale),
        _ptr(block_tables), max_blocks_per_seq, _ptr(ctx_lens), _ptr(q_lens), num_seqs, total_q,
        max_ctx_len, max_q_len, sink_tokens, window_tokens, min_ctx_len, addr, _ptr(workspace),
        workspace_bytes, _stream(stream)))
    del arr


# ---------------------------------------------------------------------------------------------
# Convenience wrapper: owns torch storage for one pool and sizes the workspace.
# ---------------------------------------------------------------------------------------------

_TORCH_DTYPE = {KV_F32: torch.float32, KV_BF16: torch.bfloat16, KV_I8: torch.int8}


class PagedKVPool:
    """A pool whose K/V storage is a pair of torch tensors on one device.

    ``k_storage`` / ``v_storage`` are flat tensors of the pool dtype (see include/kvpool.h for
    the element order); an int8 pool also owns ``k_scales`` / ``v_scales`` (float32,
    [num_layers][num_blocks][num_kv_heads][block_size]).  Metadata arguments are int32 device
    tensors.  q, out and appended rows are bf16 for an int8 pool.
    """

    def __init__(self, num_layers, num_blocks, block_size, num_kv_heads, head_dim, dtype,
                 device="cuda", k_storage=None, v_storage=None):
        self.num_layers, self.num_blocks, self.block_size = num_layers, num_blocks, block_size
        self.num_kv_heads, self.head_dim, self.dtype = num_kv_heads, head_dim, dtype
        nbytes = kvpool_storage_bytes(num_layers, num_blocks, block_size, num_kv_heads, head_dim,
                                      dtype)
        tdt = _TORCH_DTYPE[dtype]
        n = nbytes // torch.empty((), dtype=tdt).element_size()
        self.k_storage = torch.empty(n, dtype=tdt, device=device) if k_storage is None else k_storage
        self.v_storage = torch.empty(n, dtype=tdt, device=device) if v_storage is None else v_storage
        assert self.k_storage.numel() == n and self.v_storage.numel() == n
        self.k_scales = self.v_scales = None
        with torch.cuda.device(self.k_storage.device):
            if dtype == KV_I8:
                sshape = (num_layers, num_blocks, num_kv_heads, block_size)
                assert kvpool_scale_bytes(num_layers, num_blocks, block_size, num_kv_heads) == \
                    4 * num_layers * num_blocks * num_kv_heads * block_size
                self.k_scales = torch.zeros(sshape, dtype=torch.float32, device=device)
                self.v_scales = torch.zeros(sshape, dtype=torch.float32, device=device)
                self.handle = kvpool_create_int8(num_layers, num_blocks, block_size, num_kv_heads,
                                                 head_dim, self.k_storage, self.v_storage,
                                                 self.k_scales, self.v_scales)
            else:
                self.handle = kvpool_create(num_layers, num_blocks, block_size, num_kv_heads,
                                            head_dim, dtype, self.k_storage, self.v_storage)
        self._ws = None

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and _lib is not None:
            _lib.kvpool_destroy(h)
            self.handle = None

    @property
    def torch_dtype(self):
        return _TORCH_DTYPE[self.dtype]

    @property
    def act_dtype(self):
        """dtype of q, out and appended rows: the pool dtype, bf16 for an int8 pool."""
        return torch.bfloat16 if self.dtype == KV_I8 else _TORCH_DTYPE[self.dtype]

    def block_storage(self, which="k"):
        """[num_layers, num_blocks, Hkv*block_size*head_dim] view of K or V storage."""
        t = self.k_storage if which == "k" else self.v_storage
        return t.view(self.num_layers, self.num_blocks, -1)

    def append(self, layer, k_new, v_new, block_tables, ctx_lens, q_lens, max_q_len=None,
               stream=None):
        max_q_len = int(q_lens.max().item()) if max_q_len is None else max_q_len
        kvpool_append(self.handle, layer, k_new, v_new, block_tables, block_tables.shape[1],
                      ctx_lens, q_lens, ctx_lens.shape[0], k_new.shape[0], max_q_len, stream)

    def copy_blocks(self, src, dst, stream=None):
        kvpool_copy_blocks(self.handle, src, dst, src.shape[0], stream)

    def workspace(self, num_q_heads, num_seqs, total_q, max_ctx_len, max_q_len,
                  q_lens_host=None):
        need = kvattn_workspace_size(self.handle, num_q_heads, num_seqs, total_q, max_ctx_len,
                                     max_q_len, q_lens_host)
        if need and (self._ws is None or self._ws.numel() < need):
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.k_storage.device)
        return self._ws, need

    def forward(self, layer, q, block_tables, ctx_lens, q_lens, scale=None, max_ctx_len=None,
                max_q_len=None, out=None, stream=None, q_lens_host=None):
        """Attention for one call.  ``q_lens_host``: optional host copy of ``q_lens`` (list or
        numpy); with it the library sizes grids and workspace exactly."""
        total_q, hq, d = q.shape
        scale = 1.0 / math.sqrt(d) if scale is None else scale
        max_ctx_len = int(ctx_lens.max().item()) if max_ctx_len is None else max_ctx_len
        max_q_len = int(q_lens.max().item()) if max_q_len is None else max_q_len
        out = torch.empty_like(q) if out is None else out
        ws, need = self.workspace(hq, ctx_lens.shape[0], total_q, max_ctx_len, max_q_len,
                                  q_lens_host)
        kvattn_forward(self.handle, layer, q, out, hq, scale, block_tables, block_tables.shape[1],
                       ctx_lens, q_lens, ctx_lens.shape[0], total_q, max_ctx_len, max_q_len,
                       ws, need, stream, q_lens_host)
        return out

    def forward_noalloc(self, layer, q, block_tables, ctx_lens, q_lens, max_ctx_len, max_q_len,
                        out, scale=None, stream=None, q_lens_host=None):
        """forward() through kvattn_forward_noalloc: the library's static scratch instead of a
        workspace.  The caller supplies `out` and the bounds, so nothing here allocates either."""
        total_q, hq, d = q.shape
        scale = 1.0 / math.sqrt(d) if scale is None else scale
        kvattn_forward_noalloc(self.handle, layer, q, out, hq, scale, block_tables,
                               block_tables.shape[1], ctx_lens, q_lens, ctx_lens.shape[0], total_q,
                               max_ctx_len, max_q_len, stream, q_lens_host)
        return out

    def append_forward(self, layer, k_new, v_new, q, block_tables, ctx_lens, q_lens, scale=None,
                       max_ctx_len=None, max_q_len=None, out=None, stream=None, q_lens_host=None):
        """append(k_new, v_new) then forward(q) in one call (the split-K kernel writes the new
        rows itself when every sequence takes it)."""
        total_q, hq, d = q.shape
        scale = 1.0 / math.sqrt(d) if scale is None else scale
        max_ctx_len = int(ctx_lens.max().item()) if max_ctx_len is None else max_ctx_len
        max_q_len = int(q_lens.max().item()) if max_q_len is None else max_q_len
        out = torch.empty_like(q) if out is None else out
        ws, need = self.workspace(hq, ctx_lens.shape[0], total_q, max_ctx_len, max_q_len,
                                  q_lens_host)
        kvattn_append_forward(self.handle, layer, k_new, v_new, q, out, hq, scale, block_tables,
                              block_tables.shape[1], ctx_lens, q_lens, ctx_lens.shape[0], total_q,
                              max_ctx_len, max_q_len, ws, need, stream, q_lens_host)
        return out

    def forward_sparse(self, layer, q, block_tables, ctx_lens, q_lens, scale=None,
                       sink_tokens=None, window_tokens=4096, min_ctx_len=16384,
                       max_ctx_len=None, max_q_len=None, out=None, stream=None,
                       q_lens_host=None):
        """Sink + window sparse attention (decode and verification rows): a row at position p
        with p + 1 >= min_ctx_len reads only keys j < sink_tokens (default: one block) or
        j >= p + 1 - window_tokens."""
        total_q, hq, d = q.shape
        scale = 1.0 / math.sqrt(d) if scale is None else scale
        sink_tokens = self.block_size if sink_tokens is None else sink_tokens
        max_ctx_len = int(ctx_lens.max().item()) if max_ctx_len is None else max_ctx_len
        max_q_len = int(q_lens.max().item()) if max_q_len is None else max_q_len
        out = torch.empty_like(q) if out is None else out
        ws, need = self.workspace(hq, ctx_lens.shape[0], total_q, max_ctx_len, max_q_len,
                                  q_lens_host)
        kvattn_forward_sparse(self.handle, layer, q, out, hq, scale, block_tables,
                              block_tables.shape[1], ctx_lens, q_lens, ctx_lens.shape[0], total_q,
                              max_ctx_len, max_q_len, sink_tokens, window_tokens, min_ctx_len,
                              ws, need, stream, q_lens_host)
        return out

    def append_forward_sparse(self, layer, k_new, v_new, q, block_tables, ctx_lens, q_lens,
                              scale=None, sink_tokens=None, window_tokens=4096,
                              min_ctx_len=16384, max_ctx_len=None, max_q_len=None, out=None,
                              stream=None, q_lens_host=None):
        """append(k_new, v_new) then forward_sparse(q) in one call."""
        total_q, hq, d = q.shape
        scale = 1.0 / math.sqrt(d) if scale is None else scale
        sink_tokens = self.block_size if sink_tokens is None else sink_tokens
        max_ctx_len = int(ctx_lens.max().item()) if max_ctx_len is None else max_ctx_len
        max_q_len = int(q_lens.max().item()) if max_q_len is None else max_q_len
        out = torch.empty_like(q) if out is None else out
        ws, need = self.workspace(hq, ctx_lens.shape[0], total_q, max_ctx_len, max_q_len,
                                  q_lens_host)
        kvattn_append_forward_sparse(self.handle, layer, k_new, v_new, q, out, hq, scale,
                                     block_tables, block_tables.shape[1], ctx_lens, q_lens,
                                     ctx_lens.shape[0], total_q, max_ctx_len, max_q_len,
                                     sink_tokens, window_tokens, min_ctx_len, ws, need, stream,
                                     q_lens_host)
        return out


# ---------------------------------------------------------------------------------------------
# Host page store (park / restore pool blocks over PCIe, pages with equal content stored once).
# ---------------------------------------------------------------------------------------------

class HostStore:
    """A pinned host page store for the blocks of pools shaped like ``pool``."""

    def __init__(self, pool: "PagedKVPool", budget_bytes: int):
        h = _vp()
        _check(lib().kvhost_create(ctypes.byref(h), pool.handle, int(budget_bytes)))
        self.handle = h.value
        out = _sz(0)
        _check(lib().kvhost_page_bytes(pool.handle, ctypes.byref(out)))
        self.page_bytes = out.value

    def close(self):
        if getattr(self, "handle", None):
            lib().kvhost_destroy(self.handle)
            self.handle = None

    def __del__(self):  # pragma: no cover
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def _i32(x):
        return np.ascontiguousarray(np.asarray(x, dtype=np.int32))

    def park(self, pool, blocks, stream=None) -> np.ndarray:
        b = self._i32(blocks)
        ids = np.zeros(b.size, np.int64)
        _check(lib().kvhost_park(self.handle, pool.handle, b.ctypes.data, b.size, ids.ctypes.data,
                                 _stream(stream)))
        return ids

    def restore(self, pool, page_ids, dst_blocks, stream=None) -> None:
        ids = np.ascontiguousarray(np.asarray(page_ids, dtype=np.int64))
        d = self._i32(dst_blocks)
        assert ids.size == d.size
        _check(lib().kvhost_restore(self.handle, pool.handle, ids.ctypes.data, d.ctypes.data,
                                    d.size, _stream(stream)))

    def release(self, page_ids) -> None:
        ids = np.ascontiguousarray(np.asarray(page_ids, dtype=np.int64))
        _check(lib().kvhost_release(self.handle, ids.ctypes.data, ids.size))

    def stats(self):
        p, c, r = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(lib().kvhost_stats(self.handle, ctypes.byref(p), ctypes.byref(c), ctypes.byref(r)))
        return dict(pages=p.value, capacity=c.value, references=r.value)

    def page_hash(self, pool, blocks, stream=None) -> np.ndarray:
        b = self._i32(blocks)
        out = np.zeros((b.size, 2), np.uint64)
        _check(lib().kvhost_page_hash(self.handle, pool.handle, b.ctypes.data, b.size,
                                      out.ctypes.data, _stream(stream)))
        return out
