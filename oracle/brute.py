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


# ---- int8 pool --------------------------------------------------------------------------------
# Offsets of the int8 storage (per layer; t = in-block token, d = dim):
#   K: ((((b*Hkv + h)*(B/16) + t//16)*(D/16) + d//16)*16 + t%16)*16 + d%16
#   V: ((((b*Hkv + h)*(B/16) + t//16)*4 + (t%16)//4)*16 + d%16)*(D/16)*4 + (d//16)*4 + t%4
#   scale of (b, h, t): (b*Hkv + h)*B + t

def k_offset_i8(b, h, t, d, *, num_kv_heads, block_size, head_dim):
    tile, tt = divmod(t, 16)
    return (((((b * num_kv_heads + h) * (block_size // 16) + tile) * (head_dim // 16) + d // 16)
             * 16 + tt) * 16 + d % 16)


def v_offset_i8(b, h, t, d, *, num_kv_heads, block_size, head_dim):
    tile, tt = divmod(t, 16)
    return (((((b * num_kv_heads + h) * (block_size // 16) + tile) * 4 + tt // 4) * 16 + d % 16)
            * (head_dim // 16) * 4 + (d // 16) * 4 + tt % 4)


def f32(x: float) -> float:
    """Round a Python float to the nearest float32 (ties to even)."""
    import struct
    return struct.unpack("<f", struct.pack("<f", x))[0]


def quantize_row(xs):
    """One row of float32 values -> (codes, scale): s = absmax / 127 and q = rint(x / s), each
    operation rounded to float32 (a float64 quotient of float32 operands, rounded once to
    float32, is the correctly rounded float32 quotient), ties to even, clamped to +-127."""
    absmax = max(abs(x) for x in xs)
    s = f32(absmax / 127.0)
    if s == 0.0:
        return [0] * len(xs), 0.0
    return [max(-127, min(127, round(f32(x / s)))) for x in xs], s


def scatter_i8(k_codes, v_codes, k_scales, v_scales, tables, *, num_blocks, num_kv_heads,
               block_size, head_dim):
    """Flat int8 K/V storage and scale lists for one layer from dense codes k_codes[s][j][h][d]
    and scales k_scales[s][j][h]; unwritten slots hold 0."""
    n = num_blocks * num_kv_heads * block_size * head_dim
    kf, vf = [0] * n, [0] * n
    ksf = [0.0] * (num_blocks * num_kv_heads * block_size)
    vsf = [0.0] * (num_blocks * num_kv_heads * block_size)
    geo = dict(num_kv_heads=num_kv_heads, block_size=block_size, head_dim=head_dim)
    for s in range(len(k_codes)):
        for j in range(len(k_codes[s])):
            b = tables[s][j // block_size]
            t = j % block_size
            for h in range(num_kv_heads):
                ksf[(b * num_kv_heads + h) * block_size + t] = k_scales[s][j][h]
                vsf[(b * num_kv_heads + h) * block_size + t] = v_scales[s][j][h]
                for d in range(head_dim):
                    kf[k_offset_i8(b, h, t, d, **geo)] = k_codes[s][j][h][d]
                    vf[v_offset_i8(b, h, t, d, **geo)] = v_codes[s][j][h][d]
    return kf, vf, ksf, vsf


def sparse_keys(p: int, *, sink: int, window: int, min_len: int):
    """Key positions a row at absolute position p reads under sink + window sparsity, listed
    from the two ranges (the first `sink` positions, the `window` latest up to p) once p + 1
    reaches min_len; all of 0 .. p before that."""
    if p + 1 < min_len:
        return list(range(p + 1))
    head = range(min(sink, p + 1))
    tail = range(max(p + 1 - window, 0), p + 1)
    return sorted(set(head) | set(tail))


def attention_keys(q, k, v, scale, keys_of):
    """As ``attention``, but row i (absolute position p) reads only the keys keys_of(p)."""
    t_len, l_len = len(q), len(k)
    hq, hkv = len(q[0]), len(k[0])
    group = hq // hkv
    dim = len(q[0][0])
    out = []
    for i in range(t_len):
        p = l_len - t_len + i
        keys = keys_of(p)
        row = []
        for h in range(hq):
            g = h // group
            scores = [scale * math.fsum(q[i][h][d] * k[j][g][d] for d in range(dim)) for j in keys]
            m = max(scores)
            lse = m + math.log(math.fsum(math.exp(sj - m) for sj in scores))
            wts = [math.exp(sj - lse) for sj in scores]
            row.append([math.fsum(w * v[j][g][d] for w, j in zip(wts, keys)) for d in range(dim)])
        out.append(row)
    return out


def fmix64_int(k: int) -> int:
    """MurmurHash3's 64-bit finalizer on a Python int (explicit masking to 64 bits)."""
    mask = (1 << 64) - 1
    k &= mask
    k ^= k >> 33
    k = (k * 0xFF51AFD7ED558CCD) & mask
    k ^= k >> 33
    k = (k * 0xC4CEB9FE1A85EC53) & mask
    k ^= k >> 33
    return k


def unfmix64_int(k: int) -> int:
    """Inverse of fmix64_int: undo each xorshift (k ^ k >> 33 is its own inverse for a 64-bit
    word, since 2 * 33 >= 64) and each multiply (by the multiplicative inverse mod 2^64)."""
    mask = (1 << 64) - 1
    k ^= k >> 33
    k = (k * pow(0xC4CEB9FE1A85EC53, -1, 1 << 64)) & mask
    k ^= k >> 33
    k = (k * pow(0xFF51AFD7ED558CCD, -1, 1 << 64)) & mask
    k ^= k >> 33
    return k


def page_hash_bytes(data: bytes):
    """The page hash over raw bytes, word by word with struct and Python ints:
    h1 = sum fmix64(w_i + 0x9E3779B97F4A7C15 (i + 1)), h2 = sum fmix64(w_i ^ 0xD6E8FEB86659FD93 (i + 1))
    mod 2^64, w_i the i-th little-endian 64-bit word."""
    import struct
    mask = (1 << 64) - 1
    h1 = h2 = 0
    for i in range(len(data) // 8):
        (w,) = struct.unpack_from("<Q", data, 8 * i)
        h1 = (h1 + fmix64_int((w + 0x9E3779B97F4A7C15 * (i + 1)) & mask)) & mask
        h2 = (h2 + fmix64_int(w ^ ((0xD6E8FEB86659FD93 * (i + 1)) & mask))) & mask
    return h1, h2
