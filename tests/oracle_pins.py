"""Checks that pin the float64 oracle to things other than itself.

Each ``pin_*`` raises AssertionError on failure.  ``tests/test_oracle.py`` runs them against
the oracle as written; ``tests/test_oracle_mutants.py`` plants plausible mistakes in the
oracle (on the CPU) and requires that some pin catches each one.

Pins: a pure-Python brute force that scatters dense K/V into the pool (the oracle gathers);
closed forms (single key, identical keys, zero query, two keys, one-hot V, a dominant key);
invariants (GQA equals MHA with repeated KV heads, physical placement, chunked prefill over a
cached prefix equals one pass, each verification row equals a decode step at its own length,
NaN canaries in slots no table reaches).
"""
from __future__ import annotations

import math

import numpy as np

from oracle import attention as ora
from oracle import brute
from paged_kv_cache_kvpool_amd import workloads as wl

TOL = 1e-12


def _x(dtype):
    return 4 if dtype == wl.F32 else 8


def _nan_elem(dtype):
    return float("nan") if dtype == wl.F32 else int(wl.BF16_NAN)


def _as_float(vals, dtype):
    if dtype == wl.F32:
        return [float(v) for v in vals]
    return [brute.bf16_to_float(int(b)) for b in vals]


def tiny_case(seed, dtype=wl.F32, block_size=16, head_dim=8, hq=4, hkv=2, q_lens=(1, 3),
              ctx_lens=(5, 40), extra_blocks=3):
    """Dense per-sequence K/V scattered (by brute force) into a randomly placed pool."""
    rng = np.random.default_rng(seed)
    need = [(c + block_size - 1) // block_size for c in ctx_lens]
    nb = sum(need) + extra_blocks
    perm = rng.permutation(nb)
    tables = np.zeros((len(ctx_lens), max(need)), np.int32)
    pos = 0
    for s, n in enumerate(need):
        tables[s, :n] = perm[pos:pos + n]
        pos += n
    k_dense = [wl.draw(rng, (c, hkv, head_dim), dtype) for c in ctx_lens]
    v_dense = [wl.draw(rng, (c, hkv, head_dim), dtype) for c in ctx_lens]
    q = wl.draw(rng, (int(sum(q_lens)), hq, head_dim), dtype)
    kf, vf = brute.scatter([k.tolist() for k in k_dense], [v.tolist() for v in v_dense],
                           tables.tolist(), num_blocks=nb, num_kv_heads=hkv,
                           block_size=block_size, head_dim=head_dim, x=_x(dtype),
                           fill=_nan_elem(dtype))
    np_dt = np.float32 if dtype == wl.F32 else np.uint16
    shape = (1, nb, hkv * block_size * head_dim)
    return dict(dtype=dtype, block_size=block_size, head_dim=head_dim, hq=hq, hkv=hkv,
                q_lens=np.asarray(q_lens, np.int32), ctx_lens=np.asarray(ctx_lens, np.int32),
                tables=tables, q=q, k_dense=k_dense, v_dense=v_dense,
                k_pool=np.asarray(kf, dtype=np_dt).reshape(shape),
                v_pool=np.asarray(vf, dtype=np_dt).reshape(shape), num_blocks=nb,
                scale=1.0 / math.sqrt(head_dim))


def run_oracle(c, k_pool=None, v_pool=None, tables=None):
    return ora.paged_attention(c["q"], c["k_pool"] if k_pool is None else k_pool,
                               c["v_pool"] if v_pool is None else v_pool, 0,
                               c["tables"] if tables is None else tables, c["ctx_lens"],
                               c["q_lens"], scale=c["scale"], num_kv_heads=c["hkv"],
                               block_size=c["block_size"], head_dim=c["head_dim"],
                               dtype=c["dtype"])


def run_brute(c):
    dt = c["dtype"]
    rows = []
    start = 0
    for s in range(len(c["ctx_lens"])):
        t = int(c["q_lens"][s])
        q = [[_as_float(c["q"][start + i, h], dt) for h in range(c["hq"])] for i in range(t)]
        k = [[_as_float(c["k_dense"][s][j, g], dt) for g in range(c["hkv"])]
             for j in range(int(c["ctx_lens"][s]))]
        v = [[_as_float(c["v_dense"][s][j, g], dt) for g in range(c["hkv"])]
             for j in range(int(c["ctx_lens"][s]))]
        rows.extend(brute.attention(q, k, v, c["scale"]))
        start += t
    return np.asarray(rows, dtype=np.float64)


BRUTE_CASES = [
    dict(seed=1, dtype=wl.F32, block_size=16, head_dim=8, hq=4, hkv=2, q_lens=(1, 3),
         ctx_lens=(5, 40)),
    dict(seed=2, dtype=wl.BF16, block_size=16, head_dim=16, hq=4, hkv=1, q_lens=(2, 1, 4),
         ctx_lens=(2, 17, 33)),
    dict(seed=3, dtype=wl.BF16, block_size=64, head_dim=8, hq=2, hkv=2, q_lens=(4, 1),
         ctx_lens=(64, 61)),
    dict(seed=4, dtype=wl.F32, block_size=32, head_dim=16, hq=3, hkv=3, q_lens=(1, 1),
         ctx_lens=(1, 48)),
]


def pin_brute_force(**kw):
    c = tiny_case(**kw)
    o, b = run_oracle(c), run_brute(c)
    assert o.shape == b.shape
    err = float(np.max(np.abs(o - b)))
    assert err <= TOL * max(1.0, float(np.max(np.abs(b)))), err


def pin_append_matches_brute_scatter(seed=5, dtype=wl.BF16, block_size=64, head_dim=16):
    """The oracle's append of every token into a NaN pool equals the brute-force scatter,
    bit for bit (untouched slots included)."""
    c = tiny_case(seed, dtype=dtype, block_size=block_size, head_dim=head_dim, hq=2, hkv=2,
                  q_lens=(3, 5), ctx_lens=(3, 70))
    empty_k = np.full_like(c["k_pool"], _nan_elem(dtype))
    empty_v = np.full_like(c["v_pool"], _nan_elem(dtype))
    k_new = np.concatenate(c["k_dense"])
    v_new = np.concatenate(c["v_dense"])
    lens = c["ctx_lens"]
    kp, vp = ora.append(empty_k, empty_v, 0, k_new, v_new, c["tables"], lens, lens,
                        num_kv_heads=c["hkv"], block_size=block_size, head_dim=head_dim,
                        dtype=dtype)
    assert kp.tobytes() == c["k_pool"].tobytes()
    assert vp.tobytes() == c["v_pool"].tobytes()


def pin_gather_roundtrip(seed=6, dtype=wl.F32, block_size=32, head_dim=8):
    """Gathering each sequence back from the brute-force-scattered pool returns the dense bits."""
    c = tiny_case(seed, dtype=dtype, block_size=block_size, head_dim=head_dim, hq=2, hkv=2,
                  q_lens=(1, 2), ctx_lens=(31, 65))
    for s, L in enumerate(c["ctx_lens"]):
        k, v = ora.gather_kv(c["k_pool"], c["v_pool"], 0, c["tables"][s], int(L),
                             num_kv_heads=c["hkv"], block_size=block_size, head_dim=head_dim,
                             dtype=dtype)
        assert k.tobytes() == c["k_dense"][s].tobytes()
        assert v.tobytes() == c["v_dense"][s].tobytes()


def pin_copy_blocks(seed=7):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((2, 6, 40)).astype(np.float32)
    v = rng.standard_normal((2, 6, 40)).astype(np.float32)
    src, dst = [4, 0], [1, 5]
    kp, vp = ora.copy_blocks(k, v, src, dst)
    for layer in range(2):
        for blk in range(6):
            want_from = {1: 4, 5: 0}.get(blk, blk)
            for e in range(40):
                assert kp[layer, blk, e] == k[layer, want_from, e]
                assert vp[layer, blk, e] == v[layer, want_from, e]


def _dense(q, k, v, scale):
    return ora.attention(np.asarray(q, np.float64), np.asarray(k, np.float64),
                         np.asarray(v, np.float64), scale)


def pin_single_key():
    rng = np.random.default_rng(8)
    q, k, v = rng.standard_normal((1, 2, 8)), rng.standard_normal((1, 1, 8)), rng.standard_normal((1, 1, 8))
    out = _dense(q, k, v, 0.7)
    assert np.array_equal(out[0, 0], v[0, 0]) and np.array_equal(out[0, 1], v[0, 0])


def pin_identical_keys():
    """All keys equal -> each row returns the mean of the V it can see (causal rows differ)."""
    rng = np.random.default_rng(9)
    L, T = 9, 3
    k = np.repeat(rng.standard_normal((1, 1, 8)), L, axis=0)
    v = rng.standard_normal((L, 1, 8))
    q = rng.standard_normal((T, 2, 8))
    out = _dense(q, k, v, 0.35)
    for i in range(T):
        want = v[:L - T + i + 1, 0].mean(axis=0)
        assert np.max(np.abs(out[i, 0] - want)) < 1e-14
        assert np.max(np.abs(out[i, 1] - want)) < 1e-14


def pin_zero_query():
    rng = np.random.default_rng(10)
    L = 7
    k, v = rng.standard_normal((L, 2, 8)), rng.standard_normal((L, 2, 8))
    out = _dense(np.zeros((1, 4, 8)), k, v, 1.0)
    for h in range(4):
        assert np.max(np.abs(out[0, h] - v[:, h // 2].mean(axis=0))) < 1e-14


def pin_two_keys():
    rng = np.random.default_rng(11)
    q, k, v = rng.standard_normal((1, 1, 8)), rng.standard_normal((2, 1, 8)), rng.standard_normal((2, 1, 8))
    scale = 0.5
    s0 = scale * math.fsum(q[0, 0, d] * k[0, 0, d] for d in range(8))
    s1 = scale * math.fsum(q[0, 0, d] * k[1, 0, d] for d in range(8))
    sig = 1.0 / (1.0 + math.exp(-(s1 - s0)))
    want = v[0, 0] + sig * (v[1, 0] - v[0, 0])
    out = _dense(q, k, v, scale)
    assert np.max(np.abs(out[0, 0] - want)) < 1e-14


def pin_one_hot_v():
    """V[j] = e_j -> output coordinate j is the attention probability of key j."""
    rng = np.random.default_rng(12)
    L = 6
    q, k = rng.standard_normal((1, 1, 8)), rng.standard_normal((L, 1, 8))
    v = np.zeros((L, 1, 8))
    for j in range(L):
        v[j, 0, j] = 1.0
    scale = 0.9
    s = [scale * math.fsum(q[0, 0, d] * k[j, 0, d] for d in range(8)) for j in range(L)]
    z = math.fsum(math.exp(x) for x in s)
    out = _dense(q, k, v, scale)
    for j in range(L):
        assert abs(out[0, 0, j] - math.exp(s[j]) / z) < 1e-14
    assert np.all(out[0, 0, L:] == 0.0)


def pin_dominant_key():
    rng = np.random.default_rng(13)
    L = 12
    q = rng.standard_normal((1, 1, 8))
    k = rng.standard_normal((L, 1, 8)) * 0.01
    k[5, 0] = q[0, 0]
    v = rng.standard_normal((L, 1, 8))
    out = _dense(q, k, v, 1e3)
    assert np.max(np.abs(out[0, 0] - v[5, 0])) < 1e-12


def pin_gqa_equals_mha():
    rng = np.random.default_rng(14)
    T, L, hkv, grp = 3, 20, 2, 3
    q = rng.standard_normal((T, hkv * grp, 8))
    k, v = rng.standard_normal((L, hkv, 8)), rng.standard_normal((L, hkv, 8))
    out = _dense(q, k, v, 0.4)
    k_rep, v_rep = np.repeat(k, grp, axis=1), np.repeat(v, grp, axis=1)
    ref = _dense(q, k_rep, v_rep, 0.4)
    assert np.array_equal(out, ref)
    # and q-head h really reads KV head h // grp: swapping KV heads changes heads 0..grp-1
    swapped = _dense(q, k[:, ::-1], v[:, ::-1], 0.4)
    assert not np.allclose(swapped[:, :grp], out[:, :grp])


def pin_placement_invariance(seed=15):
    """Moving every block to another physical id (and fixing the tables) changes nothing."""
    c = tiny_case(seed, dtype=wl.BF16, block_size=16, head_dim=16, hq=4, hkv=2,
                  q_lens=(2, 1), ctx_lens=(30, 44))
    nb = c["num_blocks"]
    perm = np.random.default_rng(seed + 1).permutation(nb)
    k2 = np.empty_like(c["k_pool"])
    v2 = np.empty_like(c["v_pool"])
    k2[:, perm] = c["k_pool"]
    v2[:, perm] = c["v_pool"]
    t2 = perm[c["tables"]].astype(np.int32)
    a = run_oracle(c)
    b = run_oracle(c, k2, v2, t2)
    assert np.array_equal(a, b)


def pin_chunked_equals_oneshot(seed=16, prefix=37, suffix=11):
    """Suffix-only prefill over a cached prefix equals the last rows of a single pass."""
    rng = np.random.default_rng(seed)
    L = prefix + suffix
    q = rng.standard_normal((L, 4, 8))
    k, v = rng.standard_normal((L, 2, 8)), rng.standard_normal((L, 2, 8))
    full = _dense(q, k, v, 0.3)
    tail = _dense(q[prefix:], k, v, 0.3)
    assert np.max(np.abs(full[prefix:] - tail)) < TOL


def pin_verify_rows_equal_decode(seed=17, L=25, T=4):
    """Verification row i equals a single-token decode over the first L - T + i + 1 keys."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, 4, 8))
    k, v = rng.standard_normal((L, 2, 8)), rng.standard_normal((L, 2, 8))
    ver = _dense(q, k, v, 0.3)
    for i in range(T):
        n = L - T + i + 1
        dec = _dense(q[i:i + 1], k[:n], v[:n], 0.3)
        assert np.max(np.abs(ver[i] - dec[0])) < TOL


def pin_nan_canaries(seed=18):
    """Slots past ctx_len and blocks no table reaches may hold NaN; outputs stay finite."""
    c = tiny_case(seed, dtype=wl.F32, block_size=16, head_dim=8, hq=2, hkv=1, q_lens=(1, 2),
                  ctx_lens=(3, 18), extra_blocks=4)
    out = run_oracle(c)
    assert np.all(np.isfinite(out))


ALL_PINS = [
    *[(f"brute_force_{i}", pin_brute_force, kw) for i, kw in enumerate(BRUTE_CASES)],
    ("append_matches_brute_scatter", pin_append_matches_brute_scatter, {}),
    ("gather_roundtrip", pin_gather_roundtrip, {}),
    ("copy_blocks", pin_copy_blocks, {}),
    ("single_key", pin_single_key, {}),
    ("identical_keys", pin_identical_keys, {}),
    ("zero_query", pin_zero_query, {}),
    ("two_keys", pin_two_keys, {}),
    ("one_hot_v", pin_one_hot_v, {}),
    ("dominant_key", pin_dominant_key, {}),
    ("gqa_equals_mha", pin_gqa_equals_mha, {}),
    ("placement_invariance", pin_placement_invariance, {}),
    ("chunked_equals_oneshot", pin_chunked_equals_oneshot, {}),
    ("verify_rows_equal_decode", pin_verify_rows_equal_decode, {}),
    ("nan_canaries", pin_nan_canaries, {}),
]
