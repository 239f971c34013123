"""The host page store oracle (``oracle.hoststore``) against its pins (CPU only).

Pins: the page hash against a word-by-word pure-Python computation over the raw bytes
(``oracle.brute.page_hash_bytes``, struct and Python ints, no numpy); the MurmurHash3 finalizer
against its inverse; page bytes against per-layer slices taken directly from the pool arrays;
the store model's page ids against pairwise byte comparison of the pages; round trips, budget
refusals that change nothing, reference counts.  The last test plants mistakes in the oracle.
"""
import numpy as np
import pytest

from oracle import brute
from oracle import hoststore as hs
from paged_kv_cache_kvpool_amd import workloads as wl


def pools_of(w):
    if w.dtype == wl.I8:
        return (w.k_pool, w.v_pool, w.k_scales, w.v_scales)
    return (w.k_pool, w.v_pool)


def shared_prefix_case(dtype, seed=3, layers=2):
    """Three sequences whose first blocks hold the same content (a shared prefix written into
    separate blocks), plus distinct blocks."""
    w = wl.make("store_case", seed=seed, dtype=dtype, num_seqs_ctx=[64, 64, 48], q_lens=[1, 1, 1],
                num_q_heads=4, num_kv_heads=2, head_dim=64, num_layers=layers, append=False)
    pools = pools_of(w)
    t = w.block_tables
    for arr in pools:          # blocks 0-1 of sequences 1 and 2 copy those of sequence 0
        for j in range(2):
            arr[:, t[1][j]] = arr[:, t[0][j]]
            arr[:, t[2][j]] = arr[:, t[0][j]]
    return w, pools


def pin_hash(page_hash=None, n=6, seed=5):
    page_hash = page_hash or hs.page_hash
    rng = np.random.default_rng(seed)
    for k in range(n):
        data = rng.integers(0, 256, size=8 * int(rng.integers(1, 400)), dtype=np.uint8)
        if k == 0:
            data[:] = 0
        if k == 1:
            data[:] = 255
        assert page_hash(data) == brute.page_hash_bytes(data.tobytes()), k


def pin_fmix(fmix=None, seed=6):
    fmix = fmix or hs.fmix64
    rng = np.random.default_rng(seed)
    xs = rng.integers(0, 2 ** 63, size=2000, dtype=np.uint64) * np.uint64(2) + np.uint64(1)
    xs[:4] = [0, 1, 2 ** 63, 2 ** 64 - 1]
    ys = fmix(xs)
    for x, y in zip(xs.tolist(), ys.tolist()):
        assert brute.fmix64_int(x) == y
        assert brute.unfmix64_int(y) == x


def pin_page_bytes(page_bytes=None):
    page_bytes = page_bytes or hs.page_bytes
    for dtype in (wl.BF16, wl.I8, wl.F32):
        w, pools = shared_prefix_case(dtype)
        b = int(w.block_tables[0][1])
        want = b"".join(np.ascontiguousarray(arr[layer, b]).tobytes()
                        for layer in range(w.num_layers) for arr in pools)
        assert page_bytes(pools, b).tobytes() == want


def test_hash_vs_word_by_word():
    pin_hash()


def test_fmix_vs_inverse():
    pin_fmix()


def test_page_bytes_layout():
    pin_page_bytes()


def test_hash_sensitive_to_every_word():
    rng = np.random.default_rng(7)
    data = rng.integers(0, 256, size=8 * 64, dtype=np.uint8)
    base = hs.page_hash(data)
    for i in range(0, data.size, 7):
        d2 = data.copy()
        d2[i] ^= 1
        assert hs.page_hash(d2) != base, i
    swapped = data.copy().view("<u8")
    swapped[[3, 9]] = swapped[[9, 3]]
    assert hs.page_hash(swapped.view(np.uint8)) != base


@pytest.mark.parametrize("dtype", [wl.BF16, wl.I8])
def test_store_dedups_exactly_equal_pages(dtype):
    w, pools = shared_prefix_case(dtype)
    blocks = [int(b) for row in w.block_tables for b in row[:4] if b >= 0]
    st = hs.Store(capacity_pages=100)
    ids = st.park(pools, blocks)
    pbs = [hs.page_bytes(pools, b) for b in blocks]
    for i in range(len(blocks)):
        for j in range(len(blocks)):
            assert (ids[i] == ids[j]) == np.array_equal(pbs[i], pbs[j]), (i, j)
    assert len(st.pages) == len({p.tobytes() for p in pbs})
    # distinct pages have distinct hashes here
    hashes = {hs.page_hash(p) for p in pbs}
    assert len(hashes) == len(st.pages)


@pytest.mark.parametrize("dtype", [wl.BF16, wl.I8])
def test_store_round_trip_and_refcounts(dtype):
    w, pools = shared_prefix_case(dtype)
    src = [int(b) for b in w.block_tables[0][:4]]
    st = hs.Store(capacity_pages=10)
    ids = st.park(pools, src)
    dst = [int(b) for b in w.block_tables[2][:3]] + [int(w.block_tables[1][3])]
    out = st.restore(pools, ids, dst)
    for s, d in zip(src, dst):
        assert np.array_equal(hs.page_bytes(out, d), hs.page_bytes(pools, s))
    again = st.park(pools, src)
    assert again == ids and all(st.refs[i] == 2 for i in set(ids))
    st.release(ids)
    st.release(again)
    assert not st.pages and not st.refs


def test_store_budget_is_all_or_nothing():
    w, pools = shared_prefix_case(wl.BF16)
    blocks = [int(b) for b in w.block_tables[0][:4]]
    st = hs.Store(capacity_pages=3)
    assert st.park(pools, blocks) is None
    assert not st.pages
    assert st.park(pools, blocks[:3]) is not None
    assert st.park(pools, [blocks[3]]) is None          # a new page, no room
    assert st.park(pools, [blocks[0], blocks[1]]) is not None  # only hits: fits


MUTANTS = {
    "position_from_zero": lambda: _mutant_hash(start=0),
    "shift_31": lambda: _mutant_hash(shift=31),
    "big_endian": lambda: _mutant_hash(order=">u8"),
    "keys_swapped": lambda: _mutant_hash(swap=True),
}


def _mutant_hash(start=1, shift=33, order="<u8", swap=False):
    def fmix(k):
        k = k.copy()
        with np.errstate(over="ignore"):
            k ^= k >> np.uint64(shift)
            k *= hs.FMIX_C1
            k ^= k >> np.uint64(shift)
            k *= hs.FMIX_C2
            k ^= k >> np.uint64(shift)
        return k

    def page_hash(pb):
        w = np.ascontiguousarray(pb).view(order).astype(np.uint64)
        pos = np.arange(start, w.size + start, dtype=np.uint64)
        k1, k2 = (hs.KEY2, hs.KEY1) if swap else (hs.KEY1, hs.KEY2)
        with np.errstate(over="ignore"):
            a = fmix(w + k1 * pos)
            b = fmix(w ^ (k2 * pos))
        return int(a.sum(dtype=np.uint64)), int(b.sum(dtype=np.uint64))
    return page_hash


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_hash_mutants_caught(name):
    with pytest.raises(AssertionError):
        pin_hash(MUTANTS[name]())
