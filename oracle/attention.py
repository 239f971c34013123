"""float64 oracle for attention of new query tokens against a block-paged KV pool.

TEST INFRASTRUCTURE: see the package docstring.  Plain, slow and written to be checked by eye.

What is computed (the pages describe the setting, not the formula; the formula is the standard
scaled dot-product attention that every path on the pages evaluates):

* a KV pool of fixed-size token blocks shared by all sequences, each sequence owning a list of
  block ids (sparkinfer server README, "Request isolation & continuous batching" and
  "Automatic prefix cache": KV held in 16-token blocks, shared rather than copied on a prefix
  hit; NInfer serving doc, "Execution behavior": one shared pool fixed at startup);
* single-token decode for a batch of sequences (NInfer serving doc, "Execution behavior");
* verification of 1 + k draft tokens, causal among themselves (sparkinfer README, "Serve
  Qwen3.8 with DSpark"; NInfer serving doc, "Server options" --spec/--draft-tokens);
* prefix reuse, where only the uncached suffix is computed against the cached prefix and must
  agree with a single pass (sparkinfer README, "Automatic prefix cache");
* GQA: consecutive q-heads share one KV head (sparkinfer README, "Determinism": GQA-fused
  prefill attention).

Readings taken where the pages are silent: the q_len new tokens are the last q_len positions
of the ctx_len keys (bottom-right causal alignment), ctx_len counts the new tokens (their K/V
are appended first), q-head h reads KV head h // (Hq / Hkv), no soft-capping or windows.

Pool storage layout (per layer, block b, KV head h, in-block token t, dim d; X = 16 bytes /
element size, so 8 for bf16 and 4 for fp32):
    K[b][h][t // 16][d // X][t % 16][d % X]
    V[b][h][t // 16][d][t % 16]
i.e. each 16-token slice of a block holds K as 16-byte dim chunks ordered chunk-major and V
transposed (dims-major).  The gather below reads that layout with reshapes.
"""
from __future__ import annotations

import numpy as np

F32 = "f32"
BF16 = "bf16"
TILE = 16  # tokens per layout tile inside a block


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening to float64.  bf16 is given as uint16 bit patterns."""
    if dtype == F32:
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return bits.view(np.float32).astype(np.float64)


def chunk_elems(dtype: str) -> int:
    return 4 if dtype == F32 else 8


def _block_to_tokens(k_blk, v_blk, num_kv_heads, block_size, head_dim, dtype):
    """One block's raw storage -> (K, V) as [block_size, Hkv, D] in storage dtype."""
    x = chunk_elems(dtype)
    nt = block_size // TILE
    k = k_blk.reshape(num_kv_heads, nt, head_dim // x, TILE, x)
    k = k.transpose(1, 3, 0, 2, 4).reshape(block_size, num_kv_heads, head_dim)
    v = v_blk.reshape(num_kv_heads, nt, head_dim, TILE)
    v = v.transpose(1, 3, 0, 2).reshape(block_size, num_kv_heads, head_dim)
    return k, v


def gather_kv(k_pool, v_pool, layer, table_row, ctx_len, *, num_kv_heads, block_size,
              head_dim, dtype):
    """Logical K and V of one sequence, [ctx_len, Hkv, D], gathered block by block through its
    block table (bits unchanged)."""
    nblk = (int(ctx_len) + block_size - 1) // block_size
    ks, vs = [], []
    for j in range(nblk):
        b = int(table_row[j])
        k, v = _block_to_tokens(k_pool[layer, b], v_pool[layer, b], num_kv_heads, block_size,
                                head_dim, dtype)
        ks.append(k)
        vs.append(v)
    if nblk == 0:
        shape = (0, num_kv_heads, head_dim)
        return np.zeros(shape, k_pool.dtype), np.zeros(shape, v_pool.dtype)
    return np.concatenate(ks)[:ctx_len], np.concatenate(vs)[:ctx_len]


def attention(q, k, v, scale):
    """Scaled dot-product attention of T query tokens that sit at the last T of L positions.

    q: [T, Hq, D] float64; k, v: [L, Hkv, D] float64.  Returns [T, Hq, D] float64.
    Row i (absolute position L - T + i) sees keys 0 .. L - T + i.
    """
    t_len, hq, _ = q.shape
    l_len, hkv, _ = k.shape
    assert hq % hkv == 0 and 1 <= t_len <= l_len
    group = hq // hkv
    out = np.empty(q.shape, dtype=np.float64)
    pos = (l_len - t_len) + np.arange(t_len)[:, None]
    masked = np.arange(l_len)[None, :] > pos           # [T, L]
    for h in range(hq):
        g = h // group
        s = scale * (q[:, h, :] @ k[:, g, :].T)         # [T, L]
        s = np.where(masked, -np.inf, s)
        w = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h, :] = (w @ v[:, g, :]) / w.sum(axis=1, keepdims=True)
    return out


def paged_attention(q, k_pool, v_pool, layer, block_tables, ctx_lens, q_lens, *, scale,
                    num_kv_heads, block_size, head_dim, dtype, seqs=None):
    """Attention for a packed batch: q [sum(q_lens), Hq, D] (rows of sequence s contiguous, in
    sequence order).  Returns float64 [sum(q_lens), Hq, D].  ``seqs`` restricts the work to a
    subset of sequences (their rows are filled, the rest left NaN)."""
    qf = to_f64(q, dtype)
    out = np.full(qf.shape, np.nan)
    starts = np.concatenate([[0], np.cumsum(np.asarray(q_lens, dtype=np.int64))])
    todo = range(len(ctx_lens)) if seqs is None else seqs
    for s in todo:
        t_len, l_len = int(q_lens[s]), int(ctx_lens[s])
        if t_len == 0:
            continue
        k, v = gather_kv(k_pool, v_pool, layer, block_tables[s], l_len,
                         num_kv_heads=num_kv_heads, block_size=block_size, head_dim=head_dim,
                         dtype=dtype)
        rows = slice(int(starts[s]), int(starts[s]) + t_len)
        out[rows] = attention(qf[rows], to_f64(k, dtype), to_f64(v, dtype), scale)
    return out


def append(k_pool, v_pool, layer, k_new, v_new, block_tables, ctx_lens, q_lens, *,
           num_kv_heads, block_size, head_dim, dtype):
    """Pools after writing each sequence's q_len new rows at positions ctx_len - q_len ..
    ctx_len - 1 (copies; inputs untouched).  Pure integer scatter: every other bit stays."""
    kp, vp = k_pool.copy(), v_pool.copy()
    x = chunk_elems(dtype)
    row = 0
    for s in range(len(ctx_lens)):
        t_len, l_len = int(q_lens[s]), int(ctx_lens[s])
        for i in range(t_len):
            p = l_len - t_len + i
            b = int(block_tables[s][p // block_size])
            t = p % block_size
            kb = kp[layer, b].reshape(num_kv_heads, block_size // TILE, head_dim // x, TILE, x)
            vb = vp[layer, b].reshape(num_kv_heads, block_size // TILE, head_dim, TILE)
            for h in range(num_kv_heads):
                kb[h, t // TILE, :, t % TILE, :] = k_new[row + i, h].reshape(head_dim // x, x)
                vb[h, t // TILE, :, t % TILE] = v_new[row + i, h]
        row += t_len
    return kp, vp


def copy_blocks(k_pool, v_pool, src, dst):
    """Pools after pool[:, dst[i]] <- pool[:, src[i]] for every layer, K and V (copies)."""
    kp, vp = k_pool.copy(), v_pool.copy()
    for a, b in zip(src, dst):
        kp[:, int(b)] = k_pool[:, int(a)]
        vp[:, int(b)] = v_pool[:, int(a)]
    return kp, vp
