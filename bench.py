"""Benchmark of the paged-KV attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Without --workload the run measures every configuration of the hot path in one process: the
batched GQA decode (32 sequences, 1-8K keys) as the top-level fields, and the tiny fp32 decode,
the two speculative verifications (32K and 128K keys), the prefix-reuse chunked prefill and
the long-context decode (262144 + 131072 keys) under "configs", each with its own step time,
roofline (kernel and step fraction, target and whether it is met), traffic and CPU baseline.

One step is one pass of the hot path over one batch: append the new tokens' K/V into their
pool blocks (kvpool_append), then attention against the paged pool (kvattn_forward: the split
attention kernel or the prefill kernel, plus the cross-split reduce in split mode).  Inputs are
resident in HBM before the timed region.  Between steps a 1 GiB scratch read evicts the 256 MB
MALL and the L2s so every step reads its KV from HBM; that read is outside the per-step device
timings.  (A scratch *write* would leave dirty lines that the step itself must write back.)

Prints ONE JSON line.  ``value`` is the whole step's algorithmic throughput: HBM GB/s for the
decode and verify workloads (K+V of every attended token once per KV head, plus Q, O, block
tables and the appended rows), TFLOP/s for prefill (4*D per unmasked (query, key) pair per
q-head).  ``roofline`` reports the dominant kernel alone, timed with HIP events recorded by the
library around each of its launches on the launch stream; ``cpu_baseline`` times the float64
oracle on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode attention achieved HBM GB/s + KV tokens/s; prefill MFMA TFLOP/s"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
FLUSH_BYTES = 1 << 30
PCIE_PEAK_GBS = 64.0   # host link: PCIe 5.0 x16, per direction

WORKLOADS = {
    "batched_gqa_decode": dict(kind="hbm", desc="32 seqs x 1 token, ctx U[1024,8192], 32/8 heads, D=128, bf16, B=16"),
    "tiny_decode": dict(kind="latency", desc="1 seq x 1 token, ctx 256 (16 of 32 blocks), 1/1 heads, D=64, fp32"),
    "spec_verify_32k": dict(kind="hbm", desc="1 seq, 1+3 tokens causal, ctx 32768+4, 40/8 heads, D=128, bf16"),
    "spec_verify_128k": dict(kind="hbm", desc="1 seq, 1+3 tokens causal, ctx 131072+4, 40/8 heads, D=128, bf16"),
    "prefix_prefill": dict(kind="mfma", desc="4 seqs x (4096 cached + 512 new causal), 40/8 heads, D=128, bf16"),
    "long_decode": dict(kind="hbm", desc="2 seqs x 1 token at 262144 and 131072, 40/8 heads, D=128, bf16, pool 24576 blocks"),
    "mixed_step": dict(kind="hbm", desc="one call: 32 decode seqs (ctx U[1024,8192]) + 1 verify (1+3 at 32768) + "
                                        "1 prefill chunk (512 over 4096 cached), 40/8 heads, D=128, bf16"),
}
WORKLOADS["sparse_decode"] = dict(
    kind="hbm", desc="32 seqs x 1 token, ctx U[16384,65536], 32/8 heads, D=128, bf16, B=16; sink + "
                     "window sparse (first 16 + last 4096 keys)")
WORKLOADS["long_decode_sparse"] = dict(
    kind="hbm", desc="2 seqs x 1 token at 262144 and 131072, 40/8 heads, D=128, bf16; sink + window "
                     "sparse (first 16 + last 4096 keys)")
WORKLOADS["long_prefix_chunk"] = dict(
    kind="mfma", desc="1 seq x (32768 cached + 512 new causal): one chunked-prefill step of a long "
                      "prompt, 40/8 heads, D=128, bf16")
WORKLOADS["park_restore"] = dict(
    kind="pcie", desc="16 seqs x 4096 tokens sharing a 2048-token prefix (recomputed into separate "
                      "blocks), 8 layers, 8 KV heads, D=128, bf16, B=16 (512 KiB pages): park every "
                      "block in the host store (equal pages once), restore every page, release")
# The same workloads on an int8 pool (codes + one fp32 scale per token and KV head; q, out and
# appended rows bf16).
for _n in ("batched_gqa_decode", "spec_verify_32k", "spec_verify_128k", "prefix_prefill",
           "long_decode", "mixed_step", "sparse_decode"):
    WORKLOADS[_n + "_int8"] = dict(kind=WORKLOADS[_n]["kind"],
                                   desc=WORKLOADS[_n]["desc"].replace("bf16", "int8 KV (bf16 q)"))


def make_workload(name):
    from paged_kv_cache_kvpool_amd import workloads as wl
    if name.endswith("_int8"):
        base = name[:-len("_int8")]
        kw = dict(host_pool=False, dtype=wl.I8)
        if base == "batched_gqa_decode":
            return wl.batched_gqa_decode(**kw)
        if base.startswith("spec_verify_"):
            return wl.spec_verify(cached={"32k": 32768, "128k": 131072}[base.split("_")[-1]], **kw)
        if base == "prefix_prefill":
            return wl.prefix_prefill(**kw)
        if base == "long_decode":
            return wl.long_decode(**kw)
        if base == "mixed_step":
            return wl.mixed_step(**kw)
        if base == "sparse_decode":
            return wl.sparse_decode(**kw)
    if name == "sparse_decode":
        return wl.sparse_decode()
    if name == "long_decode_sparse":
        return wl.long_decode_sparse()
    if name == "batched_gqa_decode":
        return wl.batched_gqa_decode(host_pool=False)
    if name == "tiny_decode":
        return wl.tiny_decode()
    if name == "spec_verify_32k":
        return wl.spec_verify(cached=32768, host_pool=False)
    if name == "spec_verify_128k":
        return wl.spec_verify(cached=131072, host_pool=False)
    if name == "prefix_prefill":
        return wl.prefix_prefill(host_pool=False)
    if name == "long_decode":
        return wl.long_decode(host_pool=False)
    if name == "mixed_step":
        return wl.mixed_step(host_pool=False)
    if name == "long_prefix_chunk":
        return wl.long_prefix_chunk(host_pool=False)
    raise SystemExit(f"unknown workload {name}")


# Sequences with q_len * (Hq / Hkv) up to this many rows per KV head take the split-K kernel,
# longer query blocks the prefill kernel (the library's rule, stated in include/kvpool.h).
SPLIT_ROWS_MAX = 128


def attended(L, T, sparse):
    """Keys of a sequence that some query row reads (their union), and the (row, key) pairs,
    with sink + window sparsity (sink, window, min_len) or without it (None)."""
    if sparse is None:
        return L, T * (L - T) + T * (T + 1) // 2
    sink, window, min_len = sparse
    spans, pairs = [], 0
    for i in range(T):
        p = L - T + i
        if p + 1 < min_len:
            row = [(0, p + 1)]
        else:
            lo = max(0, p + 1 - window)
            row = [(0, min(sink, lo)), (lo, p + 1)]
        spans += row
        pairs += sum(b - a for a, b in row if b > a)
    keys, end = 0, 0
    for a, b in sorted(spans):
        a = max(a, end)
        if b > a:
            keys += b - a
            end = b
    return keys, pairs


def algorithmic(w):
    """Per-step algorithmic bytes and flops (and attended KV tokens), from the definition, for
    the whole step and for the sequences each attention kernel serves.  Under sink + window
    sparsity only the keys some row reads count."""
    eb = w.elt_bytes                       # pool element bytes
    ab = 4 if w.dtype == "f32" else 2      # q / out / appended row element bytes
    sb = 2 * 4 if w.dtype == "i8" else 0   # int8 pools: K and V scale per token and KV head
    d, hq, hkv = w.head_dim, w.num_q_heads, w.num_kv_heads
    g = hq // hkv
    out = dict(kv_tokens=0, kv_bytes=0, attn_bytes=0, append_bytes=0, flops=0, pairs=0,
               split_bytes=0, split_flops=0, prefill_bytes=0, prefill_flops=0)
    for L, T in zip(w.ctx_lens.astype(np.int64), w.q_lens.astype(np.int64)):
        L, T = int(L), int(T)
        keys, pairs = attended(L, T, w.sparse)          # dense: row i sees L - T + i + 1 keys
        kv = keys * hkv * (d * 2 * eb + sb)             # K and V of every key, once per KV head
        qo = 2 * T * hq * d * ab
        tab = (keys + w.block_size - 1) // w.block_size * 4
        fl = 4 * d * hq * pairs
        out["kv_tokens"] += keys
        out["kv_bytes"] += kv
        out["attn_bytes"] += kv + qo + tab
        out["pairs"] += pairs
        out["flops"] += fl
        # a kernel's own bytes: K/V, Q and the table (its output write is small beside them)
        cls = "split" if T * g <= SPLIT_ROWS_MAX else "prefill"
        out[cls + "_bytes"] += kv + T * hq * d * ab + tab
        out[cls + "_flops"] += fl
    if w.k_new is not None:  # read the new rows, write them (as codes and scales for int8)
        out["append_bytes"] = 2 * w.total_q * hkv * (d * ab + d * eb + sb // 2)
    out["step_bytes"] = out["attn_bytes"] + out["append_bytes"]
    return out


def kernel_roofline(kernel, alg, ms):
    """Roofline entry of one attention kernel: HBM-bound for the split-K and vector kernels
    (the bytes of the sequences they serve), MFMA-bound for the prefill kernel (its flops)."""
    if kernel == "attn_prefill_mfma":
        achieved = alg["prefill_flops"] / (ms * 1e-3) / 1e12
        return dict(bound="mfma", achieved=achieved, peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=achieved / MFMA_BF16_PEAK_TFLOPS)
    achieved = alg["split_bytes"] / (ms * 1e-3) / 1e9
    return dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                frac=achieved / HBM_PEAK_GBS)


def kernel_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(workload, kernel):
    """Per-launch HBM bytes from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary, or None
    when it is missing or was taken on different sources (the kernel's own file, the shared
    device helpers or the dispatcher)."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(p) as f:
            t = json.load(f)[workload]
    except (OSError, KeyError, ValueError):
        return None
    src = KERNEL_SOURCES.get(kernel)
    if t.get("kernel") != kernel or src is None or t.get("source") != src:
        return None
    try:
        if source_sha(src) != t.get("sources_sha"):
            return None
    except OSError:
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(w, dev, kind, budget_s=15.0):
    """The float64 oracle (as it stands) on a bounded sample: whole sequences, in order, until
    about budget_s of CPU work; scaled to the metric's unit.  `cores`: the BLAS threads the
    oracle's matrix products ran on."""
    from oracle import attention as ora
    from oracle import quant as oq
    from oracle import sparse as osp
    threads = blas_threads()
    geo = dict(num_kv_heads=w.num_kv_heads, block_size=w.block_size, head_dim=w.head_dim)
    i8 = w.dtype == "i8"
    if i8:
        k_pool, v_pool, k_sc, v_sc = dev.pre_append_host()
        if w.k_new is not None:
            k_pool, v_pool, k_sc, v_sc = oq.append(k_pool, v_pool, k_sc, v_sc, w.layer, w.k_new,
                                                   w.v_new, w.block_tables, w.ctx_lens, w.q_lens,
                                                   **geo)
    else:
        k_pool, v_pool = dev.pre_append_host()
        if w.k_new is not None:
            k_pool, v_pool = ora.append(k_pool, v_pool, w.layer, w.k_new, w.v_new, w.block_tables,
                                        w.ctx_lens, w.q_lens, dtype=w.dtype, **geo)
    ab = 4 if w.dtype == "f32" else 2
    per_key = w.num_kv_heads * (w.head_dim * 2 * w.elt_bytes + (8 if i8 else 0))
    n_done, t_used, b_done, f_done, tok_done = 0, 0.0, 0, 0, 0
    # whole sequences in order until the budget is spent; a workload whose every sequence takes
    # less than min_s is repeated (so that tiny workloads are timed over at least min_s)
    min_s = min(2.0, budget_s)
    order = [s for _ in range(1000) for s in range(w.num_seqs)]
    for k, s in enumerate(order):
        if k >= w.num_seqs and t_used >= min_s:
            break
        t0 = time.perf_counter()
        if w.sparse is not None:
            sink, window, min_len = w.sparse
            osp.paged_attention(w.q, k_pool, v_pool, w.layer, w.block_tables, w.ctx_lens,
                                w.q_lens, scale=w.scale, dtype=w.dtype, sink=sink, window=window,
                                min_len=min_len, scales=(k_sc, v_sc) if i8 else None, seqs=[s],
                                **geo)
        elif i8:
            oq.paged_attention(w.q, k_pool, v_pool, k_sc, v_sc, w.layer, w.block_tables,
                               w.ctx_lens, w.q_lens, scale=w.scale, seqs=[s], **geo)
        else:
            ora.paged_attention(w.q, k_pool, v_pool, w.layer, w.block_tables, w.ctx_lens,
                                w.q_lens, scale=w.scale, dtype=w.dtype, seqs=[s], **geo)
        t_used += time.perf_counter() - t0
        L, T = int(w.ctx_lens[s]), int(w.q_lens[s])
        keys, pairs = attended(L, T, w.sparse)
        n_done += 1
        tok_done += keys
        b_done += keys * per_key + 2 * T * w.num_q_heads * w.head_dim * ab
        f_done += 4 * w.head_dim * w.num_q_heads * pairs
        if t_used >= budget_s:
            break
    sample = (f"{n_done} sequence passes over {w.num_seqs} sequences ({tok_done} KV tokens, "
              f"{t_used:.2f} s of oracle time)")
    if kind == "mfma":
        return dict(value=f_done / t_used / 1e12, unit="TFLOP/s", cores=threads, kind="oracle",
                    sample=sample)
    return dict(value=b_done / t_used / 1e9, unit="GB/s", cores=threads, kind="oracle",
                sample=sample)


class Device:
    """The workload on cuda:0 through the library's binding."""

    def __init__(self, w):
        import torch
        from paged_kv_cache_kvpool_amd import binding as kb
        from paged_kv_cache_kvpool_amd import workloads as wl
        self.w = w
        self.torch = torch
        dt = {wl.BF16: kb.KV_BF16, wl.F32: kb.KV_F32, wl.I8: kb.KV_I8}[w.dtype]
        self.pool = kb.PagedKVPool(w.num_layers, w.num_blocks, w.block_size, w.num_kv_heads,
                                   w.head_dim, dt, device="cuda")
        tdt = self.pool.torch_dtype

        def dev(a, dtype):
            if a is None:
                return None
            if dtype == wl.BF16:
                return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()

        kv, vv = self.pool.block_storage("k"), self.pool.block_storage("v")
        if w.dtype == wl.I8 and w.k_pool is not None:
            kv.copy_(torch.from_numpy(w.k_pool).cuda().view(kv.shape))
            vv.copy_(torch.from_numpy(w.v_pool).cuda().view(vv.shape))
            self.pool.k_scales.copy_(torch.from_numpy(w.k_scales).cuda())
            self.pool.v_scales.copy_(torch.from_numpy(w.v_scales).cuda())
        elif w.dtype == wl.I8:
            # the workload generator's int8 recipe, drawn on the device: codes
            # round(N(0,1) * 127/4) clipped to +-127, scales 4/127 * U(0.8, 1.2), NaN scales in
            # unreferenced blocks
            g = torch.Generator(device="cuda")
            g.manual_seed(int(w.pool_seed))
            for view in (kv, vv):
                for layer in range(w.num_layers):
                    x = torch.randn(view[layer].shape, generator=g, device="cuda") * (127.0 / 4.0)
                    view[layer].copy_(x.round().clamp_(-127, 127).to(torch.int8))
            dead = torch.from_numpy(~w.referenced).cuda()
            for sc in (self.pool.k_scales, self.pool.v_scales):
                sc.copy_(torch.rand(sc.shape, generator=g, device="cuda") * 0.4 + 0.8).mul_(4.0 / 127.0)
                sc[:, dead] = float("nan")
        elif w.k_pool is not None:
            kv.copy_(dev(w.k_pool, w.dtype).view(kv.shape))
            vv.copy_(dev(w.v_pool, w.dtype).view(vv.shape))
        else:
            g = torch.Generator(device="cuda")
            g.manual_seed(int(w.pool_seed))
            for view in (kv, vv):
                for layer in range(w.num_layers):
                    view[layer].copy_(torch.randn(view[layer].shape, generator=g, device="cuda",
                                                  dtype=torch.float32).to(tdt))
                view[:, torch.from_numpy(~w.referenced).cuda()] = float("nan")
        self._pre = None
        self.q = dev(w.q, w.act_dtype)
        self.k_new, self.v_new = dev(w.k_new, w.act_dtype), dev(w.v_new, w.act_dtype)
        self.tables = torch.from_numpy(w.block_tables).cuda()
        self.ctx = torch.from_numpy(w.ctx_lens).cuda()
        self.ql = torch.from_numpy(w.q_lens).cuda()
        self.out = torch.empty_like(self.q)
        self.max_ctx, self.max_q = int(w.ctx_lens.max()), int(w.q_lens.max())
        # the serving loop knows its batch's q_lens on the host: hand the library that mirror
        self.ql_host = np.ascontiguousarray(w.q_lens, dtype=np.int32)
        self.pool.workspace(w.num_q_heads, w.num_seqs, w.total_q, self.max_ctx, self.max_q,
                            self.ql_host)

    def pre_append_host(self):
        """Host copy of the pool as drawn (taken before the first append)."""
        return self._pre

    def snapshot_pre_append(self, need):
        if not need:
            return
        from paged_kv_cache_kvpool_amd import workloads as wl
        torch = self.torch
        out = []
        for which in ("k", "v"):
            t = self.pool.block_storage(which).cpu()
            out.append(t.view(torch.int16).numpy().view(np.uint16) if self.w.dtype == wl.BF16 else t.numpy())
        if self.w.dtype == wl.I8:
            out += [self.pool.k_scales.cpu().numpy(), self.pool.v_scales.cpu().numpy()]
        self._pre = tuple(out)

    # kvattn_append_forward(_sparse) for steps with new tokens (the split-K kernel appends them
    # itself when every sequence takes it); False: kvpool_append, then the attention call.
    fused_append = True

    def step(self):
        w = self.w
        common = dict(scale=w.scale, max_ctx_len=self.max_ctx, max_q_len=self.max_q, out=self.out,
                      q_lens_host=self.ql_host)
        sp = {} if w.sparse is None else dict(zip(("sink_tokens", "window_tokens", "min_ctx_len"),
                                                  w.sparse))
        args = (w.layer,)
        if self.k_new is not None and self.fused_append:
            call = self.pool.append_forward_sparse if sp else self.pool.append_forward
            call(*args, self.k_new, self.v_new, self.q, self.tables, self.ctx, self.ql, **sp,
                 **common)
            return
        if self.k_new is not None:
            self.pool.append(w.layer, self.k_new, self.v_new, self.tables, self.ctx, self.ql,
                             max_q_len=self.max_q)
        call = self.pool.forward_sparse if sp else self.pool.forward
        call(*args, self.q, self.tables, self.ctx, self.ql, **sp, **common)


def bench_park_restore(args):
    """Park / restore over PCIe through the host page store.  One step: park the 16 sequences'
    4096 blocks (content hashes on the GPU, 2176 distinct pages copied to pinned host memory),
    restore all 4096 pages into spare blocks, release them.  Bytes counted: distinct pages
    written to the host plus pages read back."""
    import torch
    from paged_kv_cache_kvpool_amd import binding as kb
    torch.cuda.set_device(0)
    layers, hkv, d, bs, seqs, per_seq, shared = 8, 8, 128, 16, 16, 256, 128
    nb = 2 * seqs * per_seq
    t_setup = time.perf_counter()
    pool = kb.PagedKVPool(layers, nb, bs, hkv, d, kb.KV_BF16, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    for which in ("k", "v"):
        view = pool.block_storage(which)
        for layer in range(layers):
            view[layer].copy_(torch.randn(view[layer].shape, generator=g, device="cuda").to(torch.bfloat16))
    rng = np.random.default_rng(7)
    perm = rng.permutation(nb).astype(np.int32)
    tables = perm[:seqs * per_seq].reshape(seqs, per_seq)
    spare = perm[seqs * per_seq:]
    # the shared prefix: blocks 0..127 of every sequence hold sequence 0's content
    src = np.repeat(tables[0, :shared][None], seqs - 1, 0).ravel()
    dst = tables[1:, :shared].ravel()
    pool.copy_blocks(torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda())
    torch.cuda.synchronize()
    blocks = tables.ravel()
    store = kb.HostStore(pool, (shared + seqs * (per_seq - shared)) * 512 * 1024 + (64 << 20))
    page = store.page_bytes
    uniq = shared + seqs * (per_seq - shared)
    moved = uniq * page + blocks.size * page
    setup_s = time.perf_counter() - t_setup

    def step():
        ids = store.park(pool, blocks)
        store.restore(pool, ids, spare[:blocks.size])
        store.release(ids)
        return ids

    for _ in range(args.warmup):
        ids = step()
    assert store.stats()["pages"] == 0
    kb.kvpool_profile(True)
    for _ in range(args.steps):
        ids = step()
    torch.cuda.synchronize()
    kb.kvpool_profile(False)
    kt = kb.kernel_times()
    times = []
    torch.cuda.synchronize()
    t_all = time.perf_counter()
    for _ in range(args.steps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ids = step()
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
    wall = time.perf_counter() - t_all
    assert len(set(ids.tolist())) == uniq
    ms = float(np.mean(times)) * 1e3
    park_ms = kt["page_park"][1] / kt["page_park"][0]
    rest_ms = kt["page_restore"][1] / kt["page_restore"][0]
    hash_ms = kt["page_hash"][1] / kt["page_hash"][0]
    park_gbs = uniq * page / (park_ms * 1e-3) / 1e9
    rest_gbs = blocks.size * page / (rest_ms * 1e-3) / 1e9
    dom, dom_ms, dom_bytes = (("page_restore", rest_ms, blocks.size * page) if rest_ms >= park_ms
                              else ("page_park", park_ms, uniq * page))
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        cpu = park_restore_cpu(pool, blocks, spare)
    line = {
        "metric": METRIC, "value": moved / (ms * 1e-3) / 1e9, "unit": "GB/s (PCIe)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "park_restore", "desc": WORKLOADS["park_restore"]["desc"],
                   "blocks_parked": int(blocks.size), "distinct_pages": uniq, "page_bytes": page},
        "park_gbs": park_gbs, "restore_gbs": rest_gbs, "hash_ms": hash_ms,
        "park_ms": park_ms, "restore_ms": rest_ms,
        "dedup_saved_bytes": (blocks.size - uniq) * page,
        "step_ms_p10_p50_p90": [float(np.percentile(times, p)) * 1e3 for p in (10, 50, 90)],
        "kernel_ms_per_launch": {k: v[1] / v[0] for k, v in kt.items()},
        "roofline": {"bound": "pcie", "achieved": achieved, "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / PCIE_PEAK_GBS, "traffic": None, "kernel": dom,
                     "kernel_ms": dom_ms},
        "cpu_baseline": cpu, "wall_s_timed_region": wall, "setup_s": setup_s,
        "kernel_source_sha": kernel_sha(os.path.join(ROOT, "paged_kv_cache_kvpool_amd", "csrc", "kv_host.hip")),
    }
    store.close()
    print(json.dumps(line), flush=True)


def park_restore_cpu(pool, blocks, spare, budget_s=10.0):
    """The oracle's store model (byte comparison, Python dict) parking and restoring pages of
    the same pool on the host: a bounded sample of blocks, scaled to GB/s of pages moved."""
    import torch
    from oracle import hoststore as hs
    k = pool.block_storage("k").cpu().view(torch.int16).numpy()
    v = pool.block_storage("v").cpu().view(torch.int16).numpy()
    pools = (k, v)
    n, t_used, moved = 0, 0.0, 0
    step = 64
    while t_used < budget_s and n < blocks.size:
        chunk = [int(b) for b in blocks[n:n + step]]
        t0 = time.perf_counter()
        st = hs.Store(capacity_pages=10 ** 9)
        ids = st.park(pools, chunk)
        st.restore(pools, ids, [int(b) for b in spare[n:n + len(chunk)]])
        t_used += time.perf_counter() - t0
        moved += (len(st.pages) + len(chunk)) * hs.page_bytes(pools, chunk[0]).size
        n += len(chunk)
    return dict(value=moved / t_used / 1e9, unit="GB/s", cores=1, kind="oracle",
                sample=f"{n} of {blocks.size} blocks parked and restored ({t_used:.1f} s)")


# The benchmark configurations the default run measures: the headline (batched GQA decode) as
# the top-level fields, every other configuration under "configs".  Targets: decode at >= 70% of
# HBM peak, chunked prefill at >= 50% of bf16 MFMA peak; verification is reported against 70%;
# the tiny fp32 decode is a latency row (microseconds).
HEADLINE = "batched_gqa_decode"
DEFAULT_CONFIGS = ["tiny_decode", "spec_verify_32k", "spec_verify_128k", "prefix_prefill",
                   "long_decode"]
TARGETS = {"batched_gqa_decode": ("hbm", 0.70, "target"), "spec_verify_32k": ("hbm", 0.70, "aim"),
           "spec_verify_128k": ("hbm", 0.70, "aim"), "prefix_prefill": ("mfma", 0.50, "target"),
           "long_decode": ("hbm", 0.70, "target"), "tiny_decode": ("latency", None, "report us")}

# Sources whose change changes what a kernel does (its own file, the shared device helpers and
# the dispatcher that plans and launches it): the committed traffic counters of a workload count
# only while all of them hash as they did when the counters were taken.
KERNEL_SOURCES = {"attn_split_mfma": "attn_split_mfma.hip", "attn_vec": "attn_vec.hip",
                  "attn_prefill_mfma": "attn_prefill_mfma.hip"}
SHARED_SOURCES = ["common.h", "kernels.h", "kvpool.cpp"]


def source_sha(kernel_src):
    """sha256[:16] over the kernel's source and the sources it shares with the dispatcher."""
    h = hashlib.sha256()
    for f in [kernel_src] + SHARED_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_kvpool_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def cpu_info():
    """Host facts recorded beside the oracle's timing."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = os.cpu_count()
    return {"cpu_model": model, "affinity_cores": affinity,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def run_workload(wname, args, scratch, want_cpu, cpu_budget_s, single_core=False):
    """One workload: warm-up, a profiled pass (the library's HIP-event pair around every launch),
    then exactly args.steps timed steps.  Returns the JSON record (not printed)."""
    import torch
    from paged_kv_cache_kvpool_amd import binding as kb

    info = WORKLOADS[wname]
    t_setup = time.perf_counter()
    w = make_workload(wname)
    alg = algorithmic(w)
    dev = Device(w)
    dev.fused_append = not args.separate_append
    dev.snapshot_pre_append(want_cpu)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    for _ in range(args.warmup):
        dev.step()
    torch.cuda.synchronize()

    flush_f32 = scratch.view(torch.float32)

    def flush(k):
        if args.flush == "read":
            flush_f32.sum()          # reads 1 GiB: evicts with clean lines only
        elif args.flush == "write":
            scratch.fill_(k & 0xFF)  # leaves dirty lines that later reads must write back

    # Per-kernel timing: an eager pass with the library's HIP-event pairs around every launch.
    kb.kvpool_profile(True)
    for k in range(args.steps):
        flush(k)
        dev.step()
    torch.cuda.synchronize()
    kb.kvpool_profile(False)
    ktimes = kb.kernel_times()

    run = dev.step
    if args.graph:
        # Capture one step (append + attention + reduce) and replay it: the library makes no
        # host synchronisation and no memset, so the captured kernels are exactly the eager ones.
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            dev.step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            dev.step()
        run = graph.replay
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        flush(k)
        starts[k].record()
        run()
        ends[k].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    ms = float(np.mean(step_ms))

    # The dominant kernel: the attention kernel with the most time per step.
    attn_kernels = [k for k in ("attn_prefill_mfma", "attn_split_mfma", "attn_vec") if k in ktimes]
    per_step = {k: ktimes[k][1] / args.steps for k in attn_kernels}
    dom = max(attn_kernels, key=lambda k: per_step[k])
    launches, total = ktimes[dom]
    dom_ms = total / launches
    kind = info["kind"]
    if kind == "mfma":
        value, unit = alg["flops"] / (ms * 1e-3) / 1e12, "TFLOP/s"
        step_frac = value / MFMA_BF16_PEAK_TFLOPS
    else:
        value, unit = alg["step_bytes"] / (ms * 1e-3) / 1e9, "GB/s"
        step_frac = value / HBM_PEAK_GBS
    roof = kernel_roofline(dom, alg, dom_ms)
    dom_bytes = alg["prefill_bytes"] if dom == "attn_prefill_mfma" else alg["split_bytes"]
    roof["kernel"] = dom
    roof["kernel_ms"] = dom_ms
    roof["traffic"] = load_traffic(wname, dom)
    roof["step_frac"] = step_frac
    tgt = TARGETS.get(wname)
    if tgt and tgt[1] is not None:
        roof["target_frac"] = tgt[1]
        roof["target_kind"] = tgt[2]
        roof["met_kernel"] = bool(roof["frac"] >= tgt[1])
        roof["met_step"] = bool(step_frac >= tgt[1])
    # every attention kernel of the step (more than one when a call mixes sequence kinds)
    rooflines = {k: dict(kernel_roofline(k, alg, ktimes[k][1] / ktimes[k][0]),
                         kernel_ms=ktimes[k][1] / ktimes[k][0]) for k in attn_kernels}

    cpu = None
    if want_cpu:
        cpu = cpu_baseline(w, dev, kind, budget_s=cpu_budget_s)
        cpu.update(cpu_info())
        if single_core:
            try:
                from threadpoolctl import threadpool_limits
                with threadpool_limits(limits=1):
                    one = cpu_baseline(w, dev, kind, budget_s=max(2.0, cpu_budget_s / 3))
                cpu["single_core"] = {"value": one["value"], "unit": one["unit"],
                                      "sample": one["sample"]}
            except Exception as e:  # pragma: no cover
                cpu["single_core"] = {"error": str(e)}

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": unit,
        "ms_per_step": ms,
        # arithmetic types of the path: fp32 pools compute in fp32; bf16 pools on bf16 MFMA with
        # fp32 accumulation; int8 pools take q.k on the int8 matrix cores (int32 accumulation)
        # and P.V on bf16 MFMA
        "dtype": {"i8": "i8/bf16", "bf16": "bf16", "f32": "f32"}[w.dtype],
        "config": {"workload": wname, "desc": info["desc"], "kv_tokens": alg["kv_tokens"],
                   "num_seqs": w.num_seqs, "total_q": w.total_q, "block_size": w.block_size,
                   "head_dim": w.head_dim, "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
                   "kv_dtype": {"i8": "int8", "bf16": "bf16", "f32": "f32"}[w.dtype],
                   "mall_flush": args.flush, "hip_graph": bool(args.graph),
                   "append": "separate" if args.separate_append else "fused call"},
        "kv_tokens_per_s": alg["kv_tokens"] / (ms * 1e-3),
        "step_ms_p10_p50_p90": [float(np.percentile(step_ms, p)) for p in (10, 50, 90)],
        "kernel_ms_per_launch": {k: v[1] / v[0] for k, v in ktimes.items()},
        "algorithmic": {"step_bytes": alg["step_bytes"], "dominant_kernel_bytes": dom_bytes,
                        "flops": alg["flops"]},
        "roofline": roof,
        "rooflines": rooflines,
        "cpu_baseline": cpu,
        "wall_s_timed_region": wall,
        "setup_s": setup_s,
        "kernel_source_sha": source_sha(KERNEL_SOURCES[dom]),
    }
    if kind == "latency":
        rec["latency_us"] = ms * 1e3
    del dev
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None, choices=sorted(WORKLOADS),
                    help="measure this workload alone (default: the headline batched GQA decode "
                         "with every other benchmark configuration under \"configs\")")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=None,
                    help="seconds of oracle time per configuration (default 15 alone, 6 each in "
                         "the all-configuration run)")
    ap.add_argument("--graph", type=int, default=0,
                    help="1: time the step as a captured HIP graph replay (as a serving loop would; "
                         "slower than eager launches on this ROCm); 0: eager launches")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (scale for HBM counters)")
    ap.add_argument("--separate-append", action="store_true",
                    help="append with kvpool_append, then the attention call (default: one "
                         "kvattn_append_forward(_sparse) call)")
    ap.add_argument("--flush", default="read", choices=["read", "write", "none"],
                    help="evict MALL and L2 between steps by reading (default) or writing 1 GiB")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        # A plain copy of known size: reads and writes exactly 1 GiB per launch.
        src = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": FLUSH_BYTES, "launches": max(1, args.steps)}),
              flush=True)
        return
    want_cpu = not args.no_cpu_baseline
    single = args.workload is None
    wname = args.workload or HEADLINE
    if WORKLOADS[wname]["kind"] == "pcie":
        bench_park_restore(args)
        return
    scratch = torch.zeros(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    budget = args.cpu_budget if args.cpu_budget is not None else (6.0 if single else 15.0)
    t_all = time.perf_counter()
    rec = run_workload(wname, args, scratch, want_cpu, budget, single_core=single)
    line = {"metric": rec["metric"], "value": rec["value"], "unit": rec["unit"], "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": rec["ms_per_step"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": rec["dtype"], "data": "synthetic"}
    line.update({k: v for k, v in rec.items() if k not in line})
    if single:
        # every other benchmark configuration, measured in the same process the same way
        configs = {}
        for name in DEFAULT_CONFIGS:
            r = run_workload(name, args, scratch, want_cpu, budget)
            print(f"[bench] {name}: {r['value']:.4g} {r['unit']}, {r['ms_per_step'] * 1e3:.1f} us/step, "
                  f"kernel frac {r['roofline']['frac']:.3f}", file=sys.stderr, flush=True)
            configs[name] = {k: r[k] for k in ("value", "unit", "ms_per_step", "dtype", "config",
                                               "kv_tokens_per_s", "step_ms_p10_p50_p90",
                                               "kernel_ms_per_launch", "algorithmic", "roofline",
                                               "rooflines", "cpu_baseline", "wall_s_timed_region")}
            if "latency_us" in r:
                configs[name]["latency_us"] = r["latency_us"]
        line["configs"] = configs
        line["targets_met"] = {n: (c["roofline"].get("met_kernel"), c["roofline"].get("met_step"))
                               for n, c in [(wname, line)] + list(configs.items())
                               if "met_kernel" in c["roofline"]}
    line["wall_s_all_configs"] = time.perf_counter() - t_all
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
