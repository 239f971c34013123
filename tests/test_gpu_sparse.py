"""GPU parity of sink + window sparse decode / verification (kvattn_forward_sparse).

A query row at position p with p + 1 >= min_len reads only the first `sink` keys and the
`window` latest ones (sparkinfer server README, "Env", SPARKINFER_SPARSE_GQA6: the first KV block
and the last 4096 tokens once a sequence holds 16384).  Compared with ``oracle.sparse`` at the
bf16 bar; around the threshold, with verification rows on both sides of it, with parameters
that are not multiples of the 32-key chunk, with forced split sizes, on int8 pools, and at full
size.  A window that covers every context must give the dense path's bits, and each sequence
must give the same bits alone as in the batch.
"""
import sys

import numpy as np
import pytest
import torch

from paged_kv_cache_kvpool_amd import binding as kb
from paged_kv_cache_kvpool_amd import workloads as wl

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from tests.gpu_util import DeviceCase, assert_close, out_f64  # noqa: E402

PAGES = dict(sink=16, window=4096, min_len=16384)


def announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def bits(t):
    return t.detach().view(torch.int16).cpu().numpy()


@pytest.mark.parametrize("mirror", [False, True], ids=["bounds", "mirror"])
@pytest.mark.parametrize("dtype", [wl.BF16, wl.I8])
def test_sparse_decode_pages_parameters(dtype, mirror):
    announce(f"sparse decode, pages' parameters, {dtype} mirror={mirror}")
    w = wl.make(f"sparse_dec_{dtype}", seed=201, dtype=dtype,
                num_seqs_ctx=[16383, 16384, 16385, 20000, 40000, 1000, 16400],
                q_lens=[1] * 7, num_q_heads=32, num_kv_heads=8, head_dim=128)
    c = DeviceCase(w)
    c.append()
    out = c.forward_sparse(mirror=mirror, **PAGES)
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle_sparse(**PAGES), dtype, w.name, q_lens=w.q_lens)


@pytest.mark.parametrize("dtype", [wl.BF16, wl.I8])
def test_sparse_verify_around_threshold(dtype):
    """1 + 3 draft rows (G = 5: two N-tiles): at L = 16385 rows 0-1 are dense and rows 2-3
    sparse (the walk keeps every key and masks per row); from L = 16387 every row is sparse."""
    announce(f"sparse verify around the threshold, {dtype}")
    w = wl.make(f"sparse_ver_{dtype}", seed=202, dtype=dtype,
                num_seqs_ctx=[16385, 16387, 16390, 30000, 16384],
                q_lens=[4, 4, 4, 4, 4], num_q_heads=40, num_kv_heads=8, head_dim=128)
    c = DeviceCase(w)
    c.append()
    out = c.forward_sparse(**PAGES)
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle_sparse(**PAGES), dtype, w.name, q_lens=w.q_lens)


SMALL = [  # (seed, dtype, hq, hkv, d, bs, sink, window, min_len)
    (0, wl.BF16, 8, 2, 128, 16, 5, 100, 300),
    (1, wl.BF16, 5, 1, 64, 64, 0, 17, 50),
    (2, wl.BF16, 16, 2, 128, 16, 40, 1, 0),
    (3, wl.BF16, 4, 4, 64, 16, 16, 64, 64),
    (4, wl.BF16, 32, 8, 128, 64, 64, 300, 700),
    (5, wl.I8, 8, 2, 128, 16, 5, 100, 300),
    (6, wl.I8, 5, 1, 64, 64, 33, 31, 100),
    (7, wl.I8, 16, 2, 128, 16, 16, 256, 512),
    (8, wl.BF16, 10, 2, 128, 16, 3, 1000, 1),
    (9, wl.BF16, 12, 3, 64, 16, 100, 40, 150),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"s{c[0]}_{c[1]}_H{c[2]}x{c[3]}_D{c[4]}_B{c[5]}_"
                                              f"k{c[6]}w{c[7]}m{c[8]}" for c in SMALL])
def test_sparse_small_parameters(case):
    """Sink and window sizes that are not multiples of the 32-key chunk, thresholds below,
    inside and above the contexts, q_len 1 to 4, both block sizes and head dims."""
    seed, dtype, hq, hkv, d, bs, sink, window, min_len = case
    announce(f"sparse small case {case}")
    w = wl.random_case(300 + seed, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                       block_size=bs, num_seqs=6, q_len_choices=(1, 2, 3, 4), max_ctx=1500)
    c = DeviceCase(w)
    c.append()
    out = c.forward_sparse(sink, window, min_len)
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle_sparse(sink, window, min_len), dtype, w.name, q_lens=w.q_lens)


@pytest.mark.parametrize("split", ["64", "96", "4096", "12288"])
def test_sparse_forced_splits(split, monkeypatch):
    """Fixed split sizes (KVATTN_SPLIT_TOKENS): many short splits over the compressed layout,
    and splits past 2048 keys (four waves per split, merged in LDS)."""
    monkeypatch.setenv("KVATTN_SPLIT_TOKENS", split)
    announce(f"sparse forced split {split}")
    w = wl.make(f"sparse_split_{split}", seed=203, dtype=wl.BF16,
                num_seqs_ctx=[20000, 17000, 3000, 33000], q_lens=[1, 4, 2, 1],
                num_q_heads=16, num_kv_heads=4, head_dim=128)
    c = DeviceCase(w)
    c.append()
    out = c.forward_sparse(16, 2000, 5000)
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle_sparse(16, 2000, 5000), wl.BF16, w.name, q_lens=w.q_lens)


def test_sparse_without_effect_is_dense_bitwise():
    """A window that covers every context (or a threshold above every context) leaves nothing
    to skip: the sparse call gives exactly the dense call's bits."""
    announce("sparse with nothing skipped == dense")
    w = wl.make("sparse_noop", seed=204, dtype=wl.BF16, num_seqs_ctx=[3000, 700, 9000, 129],
                q_lens=[1, 4, 1, 3], num_q_heads=40, num_kv_heads=8, head_dim=128)
    c = DeviceCase(w)
    c.append()
    dense = c.forward()
    a = c.forward_sparse(16, 9000, 0)
    b = c.forward_sparse(16, 100, 9001)
    torch.cuda.synchronize()
    assert np.array_equal(bits(dense), bits(a))
    assert np.array_equal(bits(dense), bits(b))


def test_sparse_batch_invariance_bitwise():
    announce("sparse batch invariance")
    w = wl.make("sparse_inv", seed=205, dtype=wl.BF16,
                num_seqs_ctx=[17000, 700, 40000, 16386, 20000], q_lens=[1, 1, 4, 4, 2],
                num_q_heads=40, num_kv_heads=8, head_dim=128)
    c = DeviceCase(w)
    c.append()
    full = c.forward_sparse(**PAGES)
    torch.cuda.synchronize()
    starts = np.concatenate([[0], np.cumsum(w.q_lens)])
    for s in range(w.num_seqs):
        rows = slice(int(starts[s]), int(starts[s + 1]))
        sel = torch.tensor([s], device="cuda")
        alone = c.pool.forward_sparse(0, c.q[rows], c.tables[sel], c.ctx[sel], c.ql[sel],
                                      scale=w.scale, sink_tokens=16, window_tokens=4096,
                                      min_ctx_len=16384, max_ctx_len=int(w.ctx_lens[s]),
                                      max_q_len=int(w.q_lens[s]))
        torch.cuda.synchronize()
        assert np.array_equal(bits(alone), bits(full[rows])), f"sequence {s}"


def test_sparse_refuses_prefill_rows_and_fp32():
    """Refused before any launch: a call whose q_len bound allows prefill-class sequences, and
    an fp32 pool."""
    announce("sparse refusals")
    w = wl.make("sparse_refuse", seed=206, dtype=wl.BF16, num_seqs_ctx=[3000, 500],
                q_lens=[1, 300], num_q_heads=8, num_kv_heads=2, head_dim=128)
    c = DeviceCase(w)
    with pytest.raises(kb.KVPoolError) as e:
        c.forward_sparse(**PAGES)
    assert e.value.code == kb.KV_EUNSUPPORTED
    with pytest.raises(kb.KVPoolError) as e:
        c.forward_sparse(mirror=True, **PAGES)
    assert e.value.code == kb.KV_EUNSUPPORTED
    w = wl.make("sparse_refuse_f32", seed=207, dtype=wl.F32, num_seqs_ctx=[300], q_lens=[1],
                num_q_heads=2, num_kv_heads=1, head_dim=64)
    c = DeviceCase(w)
    with pytest.raises(kb.KVPoolError) as e:
        c.forward_sparse(**PAGES)
    assert e.value.code == kb.KV_EUNSUPPORTED


@pytest.mark.parametrize("dtype", [wl.BF16, wl.I8])
def test_sparse_long_decode_full(dtype):
    """The long-context decode workload (262144 and 131072 keys, pool drawn on the device) in
    the pages' sparse mode."""
    announce(f"sparse long decode full size {dtype}")
    w = wl.long_decode(dtype=dtype)
    c = DeviceCase(w)
    pools = c.host_pools()
    c.append()
    out = c.forward_sparse(mirror=True, **PAGES)
    torch.cuda.synchronize()
    if dtype == wl.I8:
        ref = c.oracle_sparse(k_pool=pools[0], v_pool=pools[1], scales=(pools[2], pools[3]), **PAGES)
    else:
        ref = c.oracle_sparse(k_pool=pools[0], v_pool=pools[1], **PAGES)
    assert_close(out_f64(out), ref, dtype, w.name)
