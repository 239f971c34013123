"""Host page store for parked KV blocks, written out plainly.

TEST INFRASTRUCTURE: see the package docstring.

The pages park evicted sequences in a pinned host-RAM budget instead of discarding them, each
taking only its real size (NInfer serving doc, "Server options", --host-kv-cache-mib), and keep
a pinned host content cache from which computed prefixes restore over PCIe, branches that share
a prefix deduplicating against the same stored pages (same section, --kv-host-cache-mib).
Readings taken (the pages give no format):

* a page is one pool block across every layer: for layer 0, 1, ...: its K bytes, its V bytes
  and, for an int8 pool, its K scale bytes and V scale bytes, each in storage order;
* two blocks are the same page when their page bytes are equal; the store keeps one copy of
  each distinct page and counts its references; a page whose count falls to zero is dropped;
* parking n blocks either stores every distinct new page or, when the budget cannot hold them,
  stores nothing (the caller falls back to recomputing, as the pages' servers do);
* restoring a page writes its bytes back into a pool block, bit for bit.

The store model below decides "same page" by comparing bytes, as the library does after its
128-bit content hash, defined in ``page_hash``, has nominated a candidate (each 64-bit
little-endian word w_i of the page, i = 0, 1, ..., is keyed by its position and passed through
the 64-bit finalizer of MurmurHash3; the two hash halves are the sums, mod 2^64, of two
differently keyed mixes).
"""
from __future__ import annotations

import numpy as np

M64 = (1 << 64) - 1
FMIX_C1 = np.uint64(0xFF51AFD7ED558CCD)   # MurmurHash3 fmix64 multipliers
FMIX_C2 = np.uint64(0xC4CEB9FE1A85EC53)
KEY1 = np.uint64(0x9E3779B97F4A7C15)      # position keys of the two halves
KEY2 = np.uint64(0xD6E8FEB86659FD93)


def page_bytes(pools, block: int) -> np.ndarray:
    """Canonical bytes of pool block `block`: pools is (K, V) or (K, V, K scales, V scales), each
    with the layer as its first axis and the block as its second."""
    parts = []
    for layer in range(pools[0].shape[0]):
        for arr in pools:
            parts.append(np.ascontiguousarray(arr[layer, block]).view(np.uint8).ravel())
    return np.concatenate(parts)


def fmix64(k: np.ndarray) -> np.ndarray:
    """MurmurHash3's 64-bit finalizer, elementwise on uint64 (wrapping multiplies)."""
    k = k.copy()
    with np.errstate(over="ignore"):
        k ^= k >> np.uint64(33)
        k *= FMIX_C1
        k ^= k >> np.uint64(33)
        k *= FMIX_C2
        k ^= k >> np.uint64(33)
    return k


def page_hash(pb: np.ndarray):
    """(h1, h2) of a page's bytes (length a multiple of 8):
    h1 = sum_i fmix64(w_i + KEY1 * (i + 1)),  h2 = sum_i fmix64(w_i ^ (KEY2 * (i + 1))),
    all mod 2^64."""
    w = np.ascontiguousarray(pb).view("<u8").astype(np.uint64)
    pos = np.arange(1, w.size + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        a = fmix64(w + KEY1 * pos)
        b = fmix64(w ^ (KEY2 * pos))
    return int(a.sum(dtype=np.uint64)), int(b.sum(dtype=np.uint64))


class Store:
    """The store's observable behaviour: page ids, their contents and reference counts."""

    def __init__(self, capacity_pages: int):
        self.capacity = capacity_pages
        self.pages = {}      # id -> bytes
        self.refs = {}       # id -> count
        self._by_content = {}
        self._next = 0

    def park(self, pools, blocks):
        """Ids for the blocks (equal pages share an id), or None when the distinct new pages do
        not fit (then nothing changes)."""
        contents = [page_bytes(pools, int(b)).tobytes() for b in blocks]
        new = {c for c in contents if c not in self._by_content}
        if len(self.pages) + len(new) > self.capacity:
            return None
        ids = []
        for c in contents:
            if c not in self._by_content:
                self._by_content[c] = self._next
                self.pages[self._next] = c
                self.refs[self._next] = 0
                self._next += 1
            pid = self._by_content[c]
            self.refs[pid] += 1
            ids.append(pid)
        return ids

    def release(self, ids):
        for pid in ids:
            self.refs[pid] -= 1
            if self.refs[pid] == 0:
                c = self.pages.pop(pid)
                del self.refs[pid]
                del self._by_content[c]

    def restore(self, pools, ids, dst_blocks):
        """Pools (copies) with page ids[i] written into block dst_blocks[i]."""
        out = [a.copy() for a in pools]
        for pid, d in zip(ids, dst_blocks):
            pb = np.frombuffer(self.pages[pid], np.uint8)
            off = 0
            for layer in range(out[0].shape[0]):
                for arr in out:
                    seg = arr[layer, int(d)]
                    n = seg.nbytes
                    arr[layer, int(d)] = pb[off:off + n].view(arr.dtype).reshape(seg.shape)
                    off += n
        return out
