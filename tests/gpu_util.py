"""Helpers for the GPU parity tests: put a seeded workload on the device, run the library
through its C ABI, and run the oracle on the same input bits."""
from __future__ import annotations

import numpy as np
import torch

from oracle import attention as ora
from oracle import quant as oq
from oracle import sparse as osp
from paged_kv_cache_kvpool_amd import binding as kb
from paged_kv_cache_kvpool_amd import workloads as wl

# int8 pools: compared with the oracle run on the exactly dequantized values, at the bf16 bar
# (q, P and out are bf16 on the GPU).
TOL = {wl.BF16: dict(max_abs=2e-2, rel_l2=5e-3), wl.F32: dict(max_abs=1e-5, rel_l2=1e-5),
       wl.I8: dict(max_abs=2e-2, rel_l2=5e-3)}
KV_DTYPE = {wl.F32: kb.KV_F32, wl.BF16: kb.KV_BF16, wl.I8: kb.KV_I8}


def to_torch(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == wl.BF16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def to_numpy(t: torch.Tensor, dtype: str) -> np.ndarray:
    t = t.detach().cpu()
    if dtype == wl.BF16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def out_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


class DeviceCase:
    """A workload materialised on the GPU (pool, q, metadata) plus its host copy."""

    def __init__(self, w: wl.Workload, device="cuda"):
        self.w = w
        self.pool = kb.PagedKVPool(w.num_layers, w.num_blocks, w.block_size, w.num_kv_heads,
                                   w.head_dim, KV_DTYPE[w.dtype], device=device)
        kview, vview = self.pool.block_storage("k"), self.pool.block_storage("v")
        if w.dtype == wl.I8 and w.k_pool is not None:
            kview.copy_(torch.from_numpy(w.k_pool).to(device).view(kview.shape))
            vview.copy_(torch.from_numpy(w.v_pool).to(device).view(vview.shape))
            self.pool.k_scales.copy_(torch.from_numpy(w.k_scales).to(device))
            self.pool.v_scales.copy_(torch.from_numpy(w.v_scales).to(device))
        elif w.dtype == wl.I8:
            # drawn on the device, with the generator's recipe (workloads.py): codes
            # round(N(0,1) * 127/4) clipped to +-127, scales 4/127 * U(0.8, 1.2), NaN scales in
            # unreferenced blocks
            g = torch.Generator(device=device)
            g.manual_seed(int(w.pool_seed))
            for view in (kview, vview):
                for layer in range(w.num_layers):
                    x = torch.randn(view[layer].shape, generator=g, device=device) * (127.0 / 4.0)
                    view[layer].copy_(x.round().clamp_(-127, 127).to(torch.int8))
            for sc in (self.pool.k_scales, self.pool.v_scales):
                sc.copy_(torch.rand(sc.shape, generator=g, device=device) * 0.4 + 0.8).mul_(4.0 / 127.0)
                if w.referenced is not None:
                    sc[:, torch.from_numpy(~w.referenced).to(device)] = float("nan")
        elif w.k_pool is not None:
            kview.copy_(to_torch(w.k_pool, w.dtype, device).view(kview.shape))
            vview.copy_(to_torch(w.v_pool, w.dtype, device).view(vview.shape))
        else:
            g = torch.Generator(device=device)
            g.manual_seed(int(w.pool_seed))
            tdt = self.pool.torch_dtype
            for view in (kview, vview):
                for layer in range(w.num_layers):
                    view[layer].copy_(torch.randn(view[layer].shape, generator=g, device=device,
                                                  dtype=torch.float32).to(tdt))
                if w.referenced is not None:
                    dead = torch.from_numpy(~w.referenced).to(device)
                    view[:, dead] = float("nan")
        act = w.act_dtype
        self.q = to_torch(w.q, act, device)
        self.tables = torch.from_numpy(w.block_tables).to(device)
        self.ctx = torch.from_numpy(w.ctx_lens).to(device)
        self.ql = torch.from_numpy(w.q_lens).to(device)
        self.k_new = None if w.k_new is None else to_torch(w.k_new, act, device)
        self.v_new = None if w.v_new is None else to_torch(w.v_new, act, device)

    # -- library --------------------------------------------------------------------------
    def append(self):
        if self.k_new is not None:
            self.pool.append(self.w.layer, self.k_new, self.v_new, self.tables, self.ctx, self.ql,
                             max_q_len=int(self.w.q_lens.max()))

    def forward(self, q=None, out=None, mirror=False):
        """Attention through the library; ``mirror``: also hand it the host copy of q_lens."""
        w = self.w
        return self.pool.forward(w.layer, self.q if q is None else q, self.tables, self.ctx,
                                 self.ql, scale=w.scale, max_ctx_len=int(w.ctx_lens.max()),
                                 max_q_len=int(w.q_lens.max()), out=out,
                                 q_lens_host=w.q_lens if mirror else None)

    def append_forward(self, out=None, mirror=False):
        """Append and attention in one call (kvattn_append_forward)."""
        w = self.w
        return self.pool.append_forward(w.layer, self.k_new, self.v_new, self.q, self.tables,
                                        self.ctx, self.ql, scale=w.scale,
                                        max_ctx_len=int(w.ctx_lens.max()),
                                        max_q_len=int(w.q_lens.max()), out=out,
                                        q_lens_host=w.q_lens if mirror else None)

    def append_forward_sparse(self, sink, window, min_len, out=None, mirror=False):
        """Append and sparse attention in one call (kvattn_append_forward_sparse)."""
        w = self.w
        return self.pool.append_forward_sparse(w.layer, self.k_new, self.v_new, self.q,
                                               self.tables, self.ctx, self.ql, scale=w.scale,
                                               sink_tokens=sink, window_tokens=window,
                                               min_ctx_len=min_len,
                                               max_ctx_len=int(w.ctx_lens.max()),
                                               max_q_len=int(w.q_lens.max()), out=out,
                                               q_lens_host=w.q_lens if mirror else None)

    # -- host copies for the oracle ---------------------------------------------------------
    def host_pools(self):
        """Host copies of the device pool: (K, V), or (K, V, K scales, V scales) for int8."""
        w = self.w
        if w.dtype == wl.I8:
            return (self.pool.block_storage("k").cpu().numpy(), self.pool.block_storage("v").cpu().numpy(),
                    self.pool.k_scales.cpu().numpy(), self.pool.v_scales.cpu().numpy())
        k = to_numpy(self.pool.block_storage("k"), w.dtype)
        v = to_numpy(self.pool.block_storage("v"), w.dtype)
        return k, v

    def oracle_pools(self, k_pool=None, v_pool=None, scales=None):
        """Host pools the oracle reads: the workload's own pre-append pool (or the given one)
        with the new rows appended by the oracle (never the device's pool).  Returns (K, V,
        scales); scales is (K scales, V scales) for int8 pools, else None."""
        w = self.w
        geo = dict(num_kv_heads=w.num_kv_heads, block_size=w.block_size, head_dim=w.head_dim)
        if k_pool is None:
            if w.k_pool is None:
                raise ValueError("pool drawn on the device: pass the pre-append host pool")
            k_pool, v_pool = w.k_pool, w.v_pool
            scales = (w.k_scales, w.v_scales) if w.dtype == wl.I8 else None
        if w.dtype == wl.I8:
            ks, vs = scales
            if w.k_new is not None:
                k_pool, v_pool, ks, vs = oq.append(k_pool, v_pool, ks, vs, w.layer, w.k_new,
                                                   w.v_new, w.block_tables, w.ctx_lens, w.q_lens,
                                                   **geo)
            return k_pool, v_pool, (ks, vs)
        if w.k_new is not None:
            k_pool, v_pool = ora.append(k_pool, v_pool, w.layer, w.k_new, w.v_new, w.block_tables,
                                        w.ctx_lens, w.q_lens, dtype=w.dtype, **geo)
        return k_pool, v_pool, None

    def oracle(self, k_pool=None, v_pool=None, seqs=None, scales=None):
        """Oracle output on the pools of ``oracle_pools``."""
        w = self.w
        k_pool, v_pool, scales = self.oracle_pools(k_pool, v_pool, scales)
        geo = dict(num_kv_heads=w.num_kv_heads, block_size=w.block_size, head_dim=w.head_dim)
        if w.dtype == wl.I8:
            return oq.paged_attention(w.q, k_pool, v_pool, scales[0], scales[1], w.layer,
                                      w.block_tables, w.ctx_lens, w.q_lens, scale=w.scale,
                                      seqs=seqs, **geo)
        return ora.paged_attention(w.q, k_pool, v_pool, w.layer, w.block_tables, w.ctx_lens,
                                   w.q_lens, scale=w.scale, dtype=w.dtype, seqs=seqs, **geo)

    def oracle_sparse(self, sink, window, min_len, k_pool=None, v_pool=None, seqs=None,
                      scales=None):
        """Sink + window sparse oracle output on the pools of ``oracle_pools``."""
        w = self.w
        k_pool, v_pool, scales = self.oracle_pools(k_pool, v_pool, scales)
        return osp.paged_attention(w.q, k_pool, v_pool, w.layer, w.block_tables, w.ctx_lens,
                                   w.q_lens, scale=w.scale, num_kv_heads=w.num_kv_heads,
                                   block_size=w.block_size, head_dim=w.head_dim, dtype=w.dtype,
                                   sink=sink, window=window, min_len=min_len, scales=scales,
                                   seqs=seqs)

    def forward_sparse(self, sink, window, min_len, q=None, out=None, mirror=False):
        """Sparse attention through the library (kvattn_forward_sparse)."""
        w = self.w
        return self.pool.forward_sparse(w.layer, self.q if q is None else q, self.tables,
                                        self.ctx, self.ql, scale=w.scale, sink_tokens=sink,
                                        window_tokens=window, min_ctx_len=min_len,
                                        max_ctx_len=int(w.ctx_lens.max()),
                                        max_q_len=int(w.q_lens.max()), out=out,
                                        q_lens_host=w.q_lens if mirror else None)


def errors(gpu: np.ndarray, ref: np.ndarray):
    mask = ~np.isnan(ref)
    d = gpu[mask] - ref[mask]
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    rel_l2 = float(np.linalg.norm(d) / max(np.linalg.norm(ref[mask]), 1e-300)) if d.size else 0.0
    return max_abs, rel_l2


# A single (row, q-head) output vector may not be off by more than this many times the
# whole-tensor rel-L2 bar: the tensor bar alone would let a few wrong vectors of a large output
# pass (one vector 20% off among 32 x 32 changes the tensor's rel-L2 by about 0.006).
VECTOR_FACTOR = 4.0


def vector_errors(gpu: np.ndarray, ref: np.ndarray):
    """Per-(row, q-head) rel-L2 of [rows, heads, D] outputs: (worst rel-L2, its (row, head),
    the rel-L2 array).  A vector's denominator is floored at 5% of the median vector norm, so a
    near-zero reference vector cannot inflate the ratio by itself."""
    g = gpu.reshape(-1, gpu.shape[-2], gpu.shape[-1]) if gpu.ndim >= 3 else gpu.reshape(-1, 1, gpu.shape[-1])
    r = ref.reshape(g.shape)
    ok = ~np.isnan(r)
    d = np.where(ok, g - r, 0.0)
    rn = np.sqrt(np.sum(np.where(ok, r, 0.0) ** 2, axis=-1))
    dn = np.sqrt(np.sum(d ** 2, axis=-1))
    floor = 0.05 * float(np.median(rn)) if rn.size else 0.0
    rel = dn / np.maximum(rn, max(floor, 1e-300))
    if rel.size == 0:
        return 0.0, (0, 0), rel
    idx = np.unravel_index(int(np.argmax(rel)), rel.shape)
    return float(rel[idx]), (int(idx[0]), int(idx[1])), rel


def row_owner(row: int, q_lens):
    """(sequence, token index within it) of packed query row `row`."""
    c = np.cumsum(np.asarray(q_lens, dtype=np.int64))
    s = int(np.searchsorted(c, row, side="right"))
    return s, int(row - (c[s - 1] if s else 0))


def assert_close(gpu: np.ndarray, ref: np.ndarray, dtype: str, what="", q_lens=None):
    """Whole-tensor max-abs and rel-L2 at the bar, and every (row, q-head) vector within
    VECTOR_FACTOR times the rel-L2 bar.  Prints the worst vector (with its sequence and token
    when q_lens is given)."""
    assert gpu.shape == ref.shape
    assert np.all(np.isfinite(gpu[~np.isnan(ref)])), f"{what}: non-finite output"
    max_abs, rel_l2 = errors(gpu, ref)
    tol = TOL[dtype]
    worst, (wr, wh), _ = vector_errors(gpu, ref)
    where = f"row {wr}, q-head {wh}"
    if q_lens is not None:
        s, i = row_owner(wr, q_lens)
        where += f" (sequence {s}, token {i})"
    print(f"[parity] {what}: max_abs={max_abs:.3e} rel_l2={rel_l2:.3e} worst vector rel_l2="
          f"{worst:.3e} at {where}", flush=True)
    assert max_abs <= tol["max_abs"] and rel_l2 <= tol["rel_l2"], \
        f"{what}: max_abs={max_abs:.3e} rel_l2={rel_l2:.3e} (tol {tol})"
    assert worst <= VECTOR_FACTOR * tol["rel_l2"], \
        f"{what}: vector at {where} has rel_l2={worst:.3e} > {VECTOR_FACTOR} x {tol['rel_l2']}"
    return max_abs, rel_l2
