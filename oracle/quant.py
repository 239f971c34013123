"""int8 KV pool: the quantisation and the attention it feeds, written out plainly.

TEST INFRASTRUCTURE: see the package docstring.

The pages store the KV cache as int8 on request (NInfer serving doc, "Server options",
--kv-dtype bf16|int8; sparkinfer server README, "Env", SPARKINFER_KV_INT8, which the server turns
on whenever the context is 4096 or more: "Determinism", known defect).  They give no scale
layout.  The reading taken here, the plainest one:

* one fp32 scale per (token, KV head), for K and for V separately: s = absmax(x) / 127, the
  absolute maximum over the row's head_dim values, computed in fp32;
* codes q = rint(x / s) in fp32 (division correctly rounded, ties to even), clamped to
  [-127, 127]; a row of zeros has s = 0 and codes 0;
* the value a code stands for is q * s; attention runs on those dequantized values (float64
  here), exactly as on a bf16 pool.

The new rows handed to the append are bf16 (the dtype of the model's K/V projections); they are
widened to fp32 exactly before quantisation.

int8 pool layout (per layer, block b, KV head h, 16-token slice t // 16 of the block):
    K tile: [d // 16][t % 16][d % 16]            16-byte chunks of 16 dims, chunk-major
    V tile: [(t % 16) // 4][d % 16][d // 16][t % 4]
(the V order puts the 4 keys t % 4 of dims d % 16, d % 16 + 16, ... side by side).  Scales:
    [b][h][t] fp32, one array for K and one for V (per layer: [num_blocks][Hkv][block_size]).
"""
from __future__ import annotations

import numpy as np

from .attention import TILE, attention, to_f64


def quantize_rows(x: np.ndarray):
    """Rows of float32 values -> (int8 codes, float32 scales), one scale per row (last axis)."""
    x = np.asarray(x, dtype=np.float32)
    absmax = np.max(np.abs(x), axis=-1)
    scale = (absmax / np.float32(127.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = np.rint((x / safe[..., None]).astype(np.float32))
    q = np.clip(q, -127, 127)
    q = np.where(scale[..., None] > 0, q, 0)
    return q.astype(np.int8), scale


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 values q * s (scales broadcast over the last axis)."""
    return codes.astype(np.float64) * np.asarray(scales, dtype=np.float64)[..., None]


def _block_codes_to_tokens(k_blk, v_blk, num_kv_heads, block_size, head_dim):
    """One block's int8 storage -> (K, V) codes as [block_size, Hkv, D]."""
    nt = block_size // TILE
    k = k_blk.reshape(num_kv_heads, nt, head_dim // 16, TILE, 16)
    k = k.transpose(1, 3, 0, 2, 4).reshape(block_size, num_kv_heads, head_dim)
    # V tile axes: [t%16 // 4][d % 16][d // 16][t % 4]  ->  [t][d]
    v = v_blk.reshape(num_kv_heads, nt, 4, 16, head_dim // 16, 4)
    v = v.transpose(1, 2, 5, 0, 4, 3).reshape(block_size, num_kv_heads, head_dim)
    return k, v


def gather_kv(k_pool, v_pool, k_scale, v_scale, layer, table_row, ctx_len, *, num_kv_heads,
              block_size, head_dim):
    """Dequantized K and V of one sequence, [ctx_len, Hkv, D] float64, gathered block by block
    through its block table.  Pools: int8 [layers][blocks][Hkv*B*D]; scales float32
    [layers][blocks][Hkv][B]."""
    nblk = (int(ctx_len) + block_size - 1) // block_size
    ks, vs = [], []
    for j in range(nblk):
        b = int(table_row[j])
        kc, vc = _block_codes_to_tokens(k_pool[layer, b], v_pool[layer, b], num_kv_heads,
                                        block_size, head_dim)
        ks.append(dequantize(kc, k_scale[layer, b].T))  # scales [B][Hkv] per token and head
        vs.append(dequantize(vc, v_scale[layer, b].T))
    if nblk == 0:
        z = np.zeros((0, num_kv_heads, head_dim))
        return z, z
    return np.concatenate(ks)[:ctx_len], np.concatenate(vs)[:ctx_len]


def paged_attention(q, k_pool, v_pool, k_scale, v_scale, layer, block_tables, ctx_lens, q_lens,
                    *, scale, num_kv_heads, block_size, head_dim, seqs=None):
    """Attention for a packed batch against an int8 pool (bf16 q given as uint16 bits).
    Returns float64 [sum(q_lens), Hq, D]."""
    qf = to_f64(q, "bf16")
    out = np.full(qf.shape, np.nan)
    starts = np.concatenate([[0], np.cumsum(np.asarray(q_lens, dtype=np.int64))])
    todo = range(len(ctx_lens)) if seqs is None else seqs
    for s in todo:
        t_len, l_len = int(q_lens[s]), int(ctx_lens[s])
        if t_len == 0:
            continue
        k, v = gather_kv(k_pool, v_pool, k_scale, v_scale, layer, block_tables[s], l_len,
                         num_kv_heads=num_kv_heads, block_size=block_size, head_dim=head_dim)
        rows = slice(int(starts[s]), int(starts[s]) + t_len)
        out[rows] = attention(qf[rows], k, v, scale)
    return out


def append(k_pool, v_pool, k_scale, v_scale, layer, k_new, v_new, block_tables, ctx_lens,
           q_lens, *, num_kv_heads, block_size, head_dim):
    """Pools and scales after quantising and writing each sequence's q_len new rows (bf16 bits
    [total_q][Hkv][D]) at positions ctx_len - q_len .. ctx_len - 1 (copies; inputs untouched)."""
    kp, vp, ks, vs = k_pool.copy(), v_pool.copy(), k_scale.copy(), v_scale.copy()
    kq, kscl = quantize_rows(to_f64(k_new, "bf16").astype(np.float32))
    vq, vscl = quantize_rows(to_f64(v_new, "bf16").astype(np.float32))
    row = 0
    for s in range(len(ctx_lens)):
        t_len, l_len = int(q_lens[s]), int(ctx_lens[s])
        for i in range(t_len):
            p = l_len - t_len + i
            b = int(block_tables[s][p // block_size])
            t = p % block_size
            kb = kp[layer, b].reshape(num_kv_heads, block_size // TILE, head_dim // 16, TILE, 16)
            vb = vp[layer, b].reshape(num_kv_heads, block_size // TILE, 4, 16, head_dim // 16, 4)
            tt = t % TILE
            for h in range(num_kv_heads):
                kb[h, t // TILE, :, tt, :] = kq[row + i, h].reshape(head_dim // 16, 16)
                # dim d = 16 * (d // 16) + d % 16  ->  [d % 16][d // 16]
                vb[h, t // TILE, tt // 4, :, :, tt % 4] = vq[row + i, h].reshape(head_dim // 16, 16).T
                ks[layer, b, h, t] = kscl[row + i, h]
                vs[layer, b, h, t] = vscl[row + i, h]
        row += t_len
    return kp, vp, ks, vs


def copy_blocks(k_pool, v_pool, k_scale, v_scale, src, dst):
    """pool[:, dst[i]] <- pool[:, src[i]] for every layer: codes and scales, K and V (copies)."""
    kp, vp, ks, vs = k_pool.copy(), v_pool.copy(), k_scale.copy(), v_scale.copy()
    for a, b in zip(src, dst):
        kp[:, int(b)] = k_pool[:, int(a)]
        vp[:, int(b)] = v_pool[:, int(a)]
        ks[:, int(b)] = k_scale[:, int(a)]
        vs[:, int(b)] = v_scale[:, int(a)]
    return kp, vp, ks, vs
