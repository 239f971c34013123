"""The sink + window sparse oracle (``oracle.sparse``) against its pins (CPU only).

Pins:
* the pure-Python brute force, which lists the keys a row reads from the two ranges instead of
  testing each key (``oracle.brute.sparse_keys`` / ``attention_keys``);
* the dense oracle run on the explicitly cut key subset (first positions + latest ones);
* reductions to dense attention, bitwise: a threshold above the context, a window covering it;
* closed forms: a window of one with no sink returns the row's own V; a one-key sink plus a
  one-key window is the two-key sigmoid blend; a one-hot V gives zero weight to every key
  outside the visible set and positive weight inside it.
The last test plants plausible mistakes in ``oracle.sparse.visible`` and requires a pin to
catch each.
"""
import math

import numpy as np
import pytest

from oracle import attention as ora
from oracle import brute
from oracle import quant as oq
from oracle import sparse as osp
from paged_kv_cache_kvpool_amd import workloads as wl


def rand_qkv(seed, t_len, l_len, hq=2, hkv=1, d=4):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((t_len, hq, d)), rng.standard_normal((l_len, hkv, d)),
            rng.standard_normal((l_len, hkv, d)))


CASES = [  # (T, L, sink, window, min_len)
    (1, 40, 4, 8, 20), (1, 40, 4, 8, 41), (1, 40, 4, 8, 40), (3, 40, 2, 6, 39),
    (4, 33, 3, 5, 31), (2, 12, 0, 1, 1), (1, 9, 9, 3, 1), (3, 20, 16, 8, 1),
    (5, 30, 1, 30, 1), (2, 25, 6, 1, 10),
]


def pin_brute(visible=None):
    for n, (t, l, sk, wn, mn) in enumerate(CASES):
        q, k, v = rand_qkv(100 + n, t, l)
        got = osp.attention(q, k, v, 0.7, sink=sk, window=wn, min_len=mn)
        want = np.array(brute.attention_keys(
            q.tolist(), k.tolist(), v.tolist(), 0.7,
            lambda p: brute.sparse_keys(p, sink=sk, window=wn, min_len=mn)))
        assert np.allclose(got, want, rtol=1e-12, atol=1e-13), (n, np.abs(got - want).max())


def pin_subset(seed=7):
    """A decode row at L >= min_len equals dense attention over [K[:sink], K[L-window:]]."""
    rng = np.random.default_rng(seed)
    for (l, sk, wn, mn) in [(300, 16, 64, 100), (300, 16, 64, 300), (129, 16, 32, 17), (80, 5, 70, 1)]:
        q = rng.standard_normal((1, 4, 8))
        k = rng.standard_normal((l, 2, 8))
        v = rng.standard_normal((l, 2, 8))
        got = osp.attention(q, k, v, 0.35, sink=sk, window=wn, min_len=mn)
        keep = sorted(set(range(min(sk, l))) | set(range(l - wn, l)))
        want = ora.attention(q, k[keep], v[keep], 0.35)
        assert np.allclose(got, want, rtol=1e-13, atol=1e-14), (l, sk, wn, mn)


def pin_closed_forms():
    q, k, v = rand_qkv(11, 4, 20, hq=3, hkv=3, d=5)
    # window of one, no sink: each row reads only its own key
    out = osp.attention(q, k, v, 1.3, sink=0, window=1, min_len=1)
    assert np.array_equal(out, np.broadcast_to(v[16:20], out.shape))
    # one sink key + a one-key window: v0 + sigmoid(s_p - s_0) (v_p - v0)
    out = osp.attention(q[-1:], k, v, 0.9, sink=1, window=1, min_len=1)
    for h in range(3):
        s0 = 0.9 * float(q[-1, h] @ k[0, h])
        sp = 0.9 * float(q[-1, h] @ k[19, h])
        sig = 1.0 / (1.0 + math.exp(-(sp - s0)))
        assert np.allclose(out[0, h], v[0, h] + sig * (v[19, h] - v[0, h]), rtol=1e-13, atol=1e-14)
    # one-hot V: the weight on key j is exactly 0 off the visible set, > 0 on it
    l = 48
    rng = np.random.default_rng(12)
    qq = rng.standard_normal((3, 1, l))
    kk = rng.standard_normal((l, 1, l)) * 0.1
    vv = np.eye(l)[:, None, :]
    w = osp.attention(qq, kk, vv, 1.0, sink=5, window=9, min_len=46)
    for i in range(3):
        p = l - 3 + i
        keys = set(brute.sparse_keys(p, sink=5, window=9, min_len=46))
        for j in range(l):
            assert (w[i, 0, j] > 0) == (j in keys), (i, j)
        assert abs(w[i, 0].sum() - 1.0) < 1e-14


def pin_dense_reductions():
    q, k, v = rand_qkv(21, 5, 60, hq=4, hkv=2, d=6)
    dense = ora.attention(q, k, v, 0.5)
    assert np.array_equal(osp.attention(q, k, v, 0.5, sink=4, window=8, min_len=61), dense)
    assert np.array_equal(osp.attention(q, k, v, 0.5, sink=0, window=60, min_len=1), dense)
    assert np.array_equal(osp.attention(q, k, v, 0.5, sink=60, window=1, min_len=1), dense)


def test_sparse_vs_brute():
    pin_brute()


def test_sparse_subset_route():
    pin_subset()


def test_sparse_closed_forms():
    pin_closed_forms()


def test_sparse_reduces_to_dense():
    pin_dense_reductions()


@pytest.mark.parametrize("dtype", [wl.BF16, wl.F32, wl.I8])
def test_sparse_paged_matches_gathered(dtype):
    """The paged wrapper gathers through the block table exactly as the dense oracle does:
    with a threshold above every context it equals the dense paged oracle bitwise, and a
    sparse decode row equals dense attention over its cut key subset."""
    w = wl.make("sp_paged", seed=41, dtype=dtype, num_seqs_ctx=[200, 90, 150], q_lens=[1, 3, 2],
                num_q_heads=4, num_kv_heads=2, head_dim=64, append=False)
    geo = dict(num_kv_heads=2, block_size=16, head_dim=64)
    sc = (w.k_scales, w.v_scales) if dtype == wl.I8 else None
    big = osp.paged_attention(w.q, w.k_pool, w.v_pool, 0, w.block_tables, w.ctx_lens, w.q_lens,
                              scale=w.scale, dtype=dtype, sink=16, window=32, min_len=10 ** 6,
                              scales=sc, **geo)
    if dtype == wl.I8:
        dense = oq.paged_attention(w.q, w.k_pool, w.v_pool, w.k_scales, w.v_scales, 0,
                                   w.block_tables, w.ctx_lens, w.q_lens, scale=w.scale, **geo)
    else:
        dense = ora.paged_attention(w.q, w.k_pool, w.v_pool, 0, w.block_tables, w.ctx_lens,
                                    w.q_lens, scale=w.scale, dtype=dtype, **geo)
    assert np.array_equal(big, dense)
    got = osp.paged_attention(w.q, w.k_pool, w.v_pool, 0, w.block_tables, w.ctx_lens, w.q_lens,
                              scale=w.scale, dtype=dtype, sink=16, window=32, min_len=100,
                              scales=sc, **geo)
    # sequence 0: one decode row at L = 200
    if dtype == wl.I8:
        k, v = oq.gather_kv(w.k_pool, w.v_pool, w.k_scales, w.v_scales, 0, w.block_tables[0], 200, **geo)
        q0 = ora.to_f64(w.q[:1], wl.BF16)
    else:
        kb, vb = ora.gather_kv(w.k_pool, w.v_pool, 0, w.block_tables[0], 200, dtype=dtype, **geo)
        k, v = ora.to_f64(kb, dtype), ora.to_f64(vb, dtype)
        q0 = ora.to_f64(w.q[:1], dtype)
    keep = list(range(16)) + list(range(168, 200))
    want = ora.attention(q0, k[keep], v[keep], w.scale)
    assert np.allclose(got[:1], want, rtol=1e-13, atol=1e-14)
    # sequence 1 (L = 90 < min_len) is dense
    assert np.array_equal(got[1:4], dense[1:4])


MUTANTS = {
    "window_one_short": lambda j, p, sink, window: (j < sink) | (j > p + 1 - window),
    "window_one_long": lambda j, p, sink, window: (j < sink) | (j >= p - window),
    "sink_one_long": lambda j, p, sink, window: (j <= sink) | (j >= p + 1 - window),
    "no_sink": lambda j, p, sink, window: j >= p + 1 - window,
}


@pytest.mark.parametrize("name", sorted(MUTANTS) + ["threshold_off_by_one"])
def test_sparse_mutants_caught(name, monkeypatch):
    def visible(p, l_len, *, sink, window, min_len):
        j = np.arange(l_len)
        seen = j <= p
        if name == "threshold_off_by_one":
            if p >= min_len:
                seen &= (j < sink) | (j >= p + 1 - window)
        elif p + 1 >= min_len:
            seen &= MUTANTS[name](j, p, sink, window)
        return seen

    monkeypatch.setattr(osp, "visible", visible)
    caught = 0
    for pin in (pin_brute, pin_subset, pin_closed_forms, pin_dense_reductions):
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, name
