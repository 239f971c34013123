"""Pure-Python brute force used to pin ``oracle.attention`` (tiny inputs only).

TEST INFRASTRUCTURE: see the package docstring.

It works in the opposite direction from the oracle: it starts from dense per-sequence K/V,
*scatters* them into a pool element by element with the storage offset formula, and computes
attention straight from the dense K/V with a log-sum-exp normalisation and ``math.fsum``.
Nothing here uses numpy.

Storage offsets (per layer; X = 16 bytes / element size; t = in-block token, d = dim):
    K: ((((b*Hkv + h)*(B/16) + t//16)*(D/X) + d//X)*16 + t%16)*X + d%X
    V: ((((b*Hkv + h)*(B/16) + t//16)*D + d)*16 + t%16
"""
from __future__ import annotations

import math


def k_offset(b, h, t, d, *, num_kv_heads, block_size, head_dim, x):
    tile, tt = divmod(t, 16)
    chunk, e = divmod(d, x)
    return (((((b * num_kv_heads + h) * (block_size // 16) + tile) * (head_dim // x) + chunk)
             * 16 + tt) * x + e)


def v_offset(b, h, t, d, *, num_kv_heads, block_size, head_dim):
    tile, tt = divmod(t, 16)
    return ((((b * num_kv_heads + h) * (block_size // 16) + tile) * head_dim + d) * 16 + tt)


def scatter(k_dense, v_dense, tables, *, num_blocks, num_kv_heads, block_size, head_dim, x,
            fill):
    """Flat K and V storage lists for one layer.  k_dense[s][j][h][d] is token j of sequence s;
    its block is tables[s][j // block_size].  Unwritten slots hold ``fill``."""
    n = num_blocks * num_kv_heads * block_size * head_dim
    kf, vf = [fill] * n, [fill] * n
    geo = dict(num_kv_heads=num_kv_heads, block_size=block_size, head_dim=head_dim)
    for s, (ks, vs) in enumerate(zip(k_dense, v_dense)):
        for j in range(len(ks)):
            b = tables[s][j // block_size]
            t = j % block_size
            for h in range(num_kv_heads):
                for d in range(head_dim):
                    kf[k_offset(b, h, t, d, x=x, **geo)] = ks[j][h][d]
                    vf[v_offset(b, h, t, d, **geo)] = vs[j][h][d]
    return kf, vf


def attention(q, k, v, scale):
    """q[i][h][d] for T query rows at the last T of L positions; k[j][g][d], v[j][g][d] dense.
    Returns out[i][h][d] as nested lists of float."""
    t_len, l_len = len(q), len(k)
    hq, hkv = len(q[0]), len(k[0])
    group = hq // hkv
    dim = len(q[0][0])
    out = []
    for i in range(t_len):
        p = l_len - t_len + i
        row = []
        for h in range(hq):
            g = h // group
            scores = [scale * math.fsum(q[i][h][d] * k[j][g][d] for d in range(dim))
                      for j in range(p + 1)]
            m = max(scores)
            lse = m + math.log(math.fsum(math.exp(sj - m) for sj in scores))
            wts = [math.exp(sj - lse) for sj in scores]
            row.append([math.fsum(wts[j] * v[j][g][d] for j in range(p + 1))
                        for d in range(dim)])
        out.append(row)
    return out


def bf16_to_float(bits: int) -> float:
    """Exact value of a bf16 bit pattern (the top 16 bits of a float32)."""
    import struct
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]
