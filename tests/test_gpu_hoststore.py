"""GPU parity of the host page store (park / restore of pool blocks over PCIe).

The page hashes computed on the GPU equal ``oracle.hoststore.page_hash`` bit for bit; park gives
two blocks the same page id exactly when their page bytes are equal (the oracle store model
decides by comparing bytes); restore writes pages back bit for bit (whole pool compared with the
oracle store's result); the budget rule is all or nothing; releases and stale ids follow the
reference counts.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import hoststore as hs
from paged_kv_cache_kvpool_amd import binding as kb
from paged_kv_cache_kvpool_amd import workloads as wl

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from tests.gpu_util import DeviceCase  # noqa: E402


def announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def host_pools_of(w):
    return (w.k_pool, w.v_pool, w.k_scales, w.v_scales) if w.dtype == wl.I8 else (w.k_pool, w.v_pool)


def shared_case(dtype, seed=11, layers=3, block_size=16, head_dim=128, kv_heads=2):
    """Four sequences whose first two blocks hold the same content (a prefix recomputed into
    separate blocks), the rest distinct; spare blocks for restores."""
    w = wl.make("store_gpu", seed=seed, dtype=dtype, num_seqs_ctx=[100, 90, 70, 40],
                q_lens=[1, 1, 1, 1], num_q_heads=2 * kv_heads, num_kv_heads=kv_heads,
                head_dim=head_dim, block_size=block_size, num_layers=layers, append=False,
                num_blocks=(4 * 112 // block_size) + 40)
    t = w.block_tables
    nblk = [(int(c) + block_size - 1) // block_size for c in w.ctx_lens]
    for arr in host_pools_of(w):
        for s in (1, 2, 3):
            for j in range(min(2, nblk[s])):
                arr[:, t[s][j]] = arr[:, t[0][j]]
    blocks = [int(t[s][j]) for s in range(4) for j in range(nblk[s])]
    spare = [b for b in range(w.num_blocks) if b not in set(blocks)]
    return w, blocks, spare


@pytest.mark.parametrize("dtype,layers,bs,d", [(wl.BF16, 3, 16, 128), (wl.I8, 2, 64, 64),
                                               (wl.F32, 1, 16, 64), (wl.BF16, 1, 64, 128)])
def test_page_hash_bitexact(dtype, layers, bs, d):
    announce(f"page hash {dtype} layers={layers} B={bs} D={d}")
    w, blocks, _ = shared_case(dtype, layers=layers, block_size=bs, head_dim=d)
    c = DeviceCase(w)
    store = kb.HostStore(c.pool, 1 << 24)
    got = store.page_hash(c.pool, blocks)
    pools = host_pools_of(w)
    for j, b in enumerate(blocks):
        assert tuple(int(x) for x in got[j]) == hs.page_hash(hs.page_bytes(pools, b)), (j, b)
    store.close()


@pytest.mark.parametrize("dtype", [wl.BF16, wl.I8, wl.F32])
def test_park_restore_round_trip(dtype):
    announce(f"park / restore {dtype}")
    w, blocks, spare = shared_case(dtype)
    c = DeviceCase(w)
    store = kb.HostStore(c.pool, 64 << 20)
    ids = store.park(c.pool, blocks)
    pools = host_pools_of(w)
    model = hs.Store(capacity_pages=10 ** 6)
    mids = model.park(pools, blocks)
    # same page id exactly where the oracle's byte comparison says the pages are equal
    for i in range(len(blocks)):
        for j in range(len(blocks)):
            assert (ids[i] == ids[j]) == (mids[i] == mids[j]), (i, j)
    st = store.stats()
    assert st["pages"] == len(model.pages) and st["references"] == len(blocks)
    # restore every parked block into spare blocks; the whole pool must match the oracle's
    dst = spare[:len(blocks)]
    store.restore(c.pool, ids, dst)
    torch.cuda.synchronize()
    want = model.restore(pools, mids, dst)
    got = c.host_pools()
    for g, x in zip(got, want):
        assert np.array_equal(np.asarray(g).view(np.uint8), np.asarray(x).view(np.uint8))
    store.release(ids)
    assert store.stats() == dict(pages=0, capacity=st["capacity"], references=0)
    store.close()


@pytest.mark.parametrize("bits", [0, 2])
def test_forced_hash_collisions_keep_pages_apart(bits, monkeypatch):
    """With the hash cut to `bits` bits (a test knob of the library), distinct pages collide; the
    GPU byte comparison must still keep them apart, across two park calls (the second call's
    blocks meet stored pages), and restores must be bit exact."""
    announce(f"forced hash collisions, {bits} hash bits")
    monkeypatch.setenv("KVHOST_HASH_BITS", str(bits))
    w, blocks, spare = shared_case(wl.BF16, layers=2)
    c = DeviceCase(w)
    store = kb.HostStore(c.pool, 64 << 20)
    pools = host_pools_of(w)
    model = hs.Store(capacity_pages=10 ** 6)
    half = len(blocks) // 2
    ids = list(store.park(c.pool, blocks[:half])) + list(store.park(c.pool, blocks[half:]))
    mids = model.park(pools, blocks[:half]) + model.park(pools, blocks[half:])
    for i in range(len(blocks)):
        for j in range(len(blocks)):
            assert (ids[i] == ids[j]) == (mids[i] == mids[j]), (i, j)
    assert store.stats()["pages"] == len(model.pages)
    dst = spare[:len(blocks)]
    store.restore(c.pool, np.array(ids, dtype=np.int64), dst)
    torch.cuda.synchronize()
    want = model.restore(pools, mids, dst)
    for g, x in zip(c.host_pools(), want):
        assert np.array_equal(np.asarray(g).view(np.uint8), np.asarray(x).view(np.uint8))
    store.close()


def test_restore_into_another_pool():
    """Pages parked from one pool restore into another pool of the same geometry."""
    announce("restore into another pool")
    w, blocks, spare = shared_case(wl.BF16, layers=2)
    a = DeviceCase(w)
    w2, _, _ = shared_case(wl.BF16, layers=2, seed=99)
    b = DeviceCase(w2)
    store = kb.HostStore(a.pool, 64 << 20)
    ids = store.park(a.pool, blocks[:5])
    store.restore(b.pool, ids, spare[:5])
    torch.cuda.synchronize()
    pa, pb = host_pools_of(w), b.host_pools()
    for s, d in zip(blocks[:5], spare[:5]):
        assert np.array_equal(hs.page_bytes(pb, d), hs.page_bytes(pa, s))
    store.close()


def test_budget_is_all_or_nothing():
    announce("store budget")
    w, blocks, _ = shared_case(wl.BF16, layers=2)
    c = DeviceCase(w)
    page = kb.HostStore(c.pool, 1 << 24).page_bytes
    stride = (page + 255) // 256 * 256
    store = kb.HostStore(c.pool, 3 * stride + 100)     # room for 3 pages
    assert store.stats()["capacity"] == 3
    with pytest.raises(kb.KVPoolError) as e:
        store.park(c.pool, blocks[:5])                 # 5 distinct pages
    assert e.value.code == kb.KV_ENOMEM
    assert store.stats() == dict(pages=0, capacity=3, references=0)
    ids = store.park(c.pool, blocks[:3])
    with pytest.raises(kb.KVPoolError):
        store.park(c.pool, [blocks[3]])
    assert store.stats() == dict(pages=3, capacity=3, references=3)
    again = store.park(c.pool, blocks[:2])             # stored pages only: fits
    assert list(again) == list(ids[:2])
    store.close()


def test_release_and_stale_ids():
    announce("release and stale ids")
    w, blocks, spare = shared_case(wl.BF16, layers=1)
    c = DeviceCase(w)
    store = kb.HostStore(c.pool, 1 << 24)
    ids = store.park(c.pool, blocks[:4])
    with pytest.raises(kb.KVPoolError) as e:
        store.release([ids[0], ids[0]])                # one reference only
    assert e.value.code == kb.KV_EINVAL
    assert store.stats()["references"] == 4            # nothing released
    store.release(ids[:1])
    with pytest.raises(kb.KVPoolError) as e:
        store.restore(c.pool, ids[:1], spare[:1])      # stale id
    assert e.value.code == kb.KV_EINVAL
    with pytest.raises(kb.KVPoolError) as e:
        store.restore(c.pool, ids[1:3], [spare[0], spare[0]])  # duplicate destination
    assert e.value.code == kb.KV_EINVAL
    with pytest.raises(kb.KVPoolError) as e:
        store.park(c.pool, [w.num_blocks])             # outside the pool
    assert e.value.code == kb.KV_ERANGE
    # the freed slot is reused by a new page under a new id; the old id stays stale
    new = store.park(c.pool, [blocks[5]])
    assert new[0] != ids[0] and (int(new[0]) & 0xffffffff) == (int(ids[0]) & 0xffffffff)
    with pytest.raises(kb.KVPoolError):
        store.release(ids[:1])
    store.close()


def test_many_pages():
    """Several thousand pages in one park and one restore."""
    announce("many pages")
    w = wl.make("store_many", seed=12, dtype=wl.BF16, num_seqs_ctx=[16 * 1500, 16 * 1500],
                q_lens=[1, 1], num_q_heads=8, num_kv_heads=8, head_dim=128, num_layers=2,
                append=False, num_blocks=3200)
    c = DeviceCase(w)
    store = kb.HostStore(c.pool, 1 << 31)
    blocks = [int(b) for b in w.block_tables[0][:1500]]
    ids = store.park(c.pool, blocks)
    assert store.stats()["pages"] == 1500
    dst = [int(b) for b in w.block_tables[1][:1500]]
    store.restore(c.pool, ids, dst)
    torch.cuda.synchronize()
    got = c.host_pools()
    pools = host_pools_of(w)
    for s, d in zip(blocks[::37], dst[::37]):
        assert np.array_equal(hs.page_bytes(got, d), hs.page_bytes(pools, s))
    h = store.page_hash(c.pool, dst)
    for j in range(0, 1500, 101):
        assert tuple(int(x) for x in h[j]) == hs.page_hash(hs.page_bytes(pools, blocks[j]))
    store.close()
