"""GPU parity of kvattn_append_forward (append and attention in one call): the output and the
whole pool after the call equal, bit for bit, those of kvpool_append followed by kvattn_forward
on an identical second pool, and the output matches the oracle.  On bf16 pools the split-K
kernel appends when every sequence takes it (decode, verification, many sequences, new tokens on
both sides of a split boundary), on int8 pools when every sequence also runs in 32-row tiles
(verification); calls with prefill chunks, 16-row int8 calls, fp32 pools and the vector path use
the append kernel.  kvattn_append_forward_sparse is held to the same bar against kvpool_append
followed by kvattn_forward_sparse (sequences below and above the sparse threshold, new tokens
past the skipped keys, fixed splits that cut the window) and against the sparse oracle.
"""
import sys

import numpy as np
import pytest
import torch

from paged_kv_cache_kvpool_amd import workloads as wl

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from tests.gpu_util import DeviceCase, assert_close, out_f64  # noqa: E402


def announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def raw(t):
    return t.detach().contiguous().view(torch.uint8).cpu().numpy()


CASES = {
    "decode": dict(num_seqs_ctx=[3000, 700, 40, 9000, 17, 256, 257], q_lens=[1] * 7,
                   num_q_heads=32, num_kv_heads=8),
    "verify": dict(num_seqs_ctx=[32772, 2050, 4], q_lens=[4, 4, 4], num_q_heads=40, num_kv_heads=8),
    "many": dict(num_seqs_ctx=list(range(300, 300 + 97 * 37, 37)), q_lens=[1, 2, 1, 4] * 24 + [1],
                 num_q_heads=16, num_kv_heads=4),
    "mixed": dict(num_seqs_ctx=[3000, 700, 900, 5000], q_lens=[1, 4, 300, 1], num_q_heads=40,
                  num_kv_heads=8),
    "wide_rows": dict(num_seqs_ctx=[5000, 1300], q_lens=[8, 5], num_q_heads=64, num_kv_heads=8),
    # three prefill sequences (two whole prompts) beside decode and verification, 64-token blocks
    "mixed_prompts": dict(num_seqs_ctx=[1200, 64, 2049, 700, 33, 5000], q_lens=[1, 64, 129, 4, 33, 1],
                          num_q_heads=32, num_kv_heads=8, block_size=64),
}


def pair(name, dtype, seed):
    cfg = CASES[name]
    w = wl.make(f"af_{name}_{dtype}", seed=seed, dtype=dtype, head_dim=128, **cfg)
    return w, DeviceCase(w), DeviceCase(w)


def check(name, dtype, seed=601, mirror=True):
    announce(f"append_forward {name} {dtype} mirror={mirror}")
    w, a, b = pair(name, dtype, seed)
    a.append()
    ref = a.forward(mirror=mirror)
    got = b.append_forward(mirror=mirror)
    torch.cuda.synchronize()
    assert np.array_equal(raw(got), raw(ref)), "output differs from append + forward"
    for x, y in zip(a.host_pools(), b.host_pools()):
        assert np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8)), \
            "pool differs from append + forward"
    assert_close(out_f64(got), b.oracle(), dtype, w.name, q_lens=w.q_lens)


@pytest.mark.parametrize("name", ["decode", "verify", "many", "wide_rows", "mixed", "mixed_prompts"])
@pytest.mark.parametrize("dtype", [wl.BF16, wl.I8])
def test_append_forward(name, dtype):
    check(name, dtype)


def test_append_forward_without_mirror():
    check("verify", wl.BF16, mirror=False)
    check("decode", wl.I8, mirror=False)
    check("mixed", wl.BF16, mirror=False)
    check("mixed_prompts", wl.BF16, mirror=False)


@pytest.mark.parametrize("dtype", [wl.BF16, wl.I8])
@pytest.mark.parametrize("split", ["256", "512"])
def test_new_tokens_across_a_split_boundary(split, dtype, monkeypatch):
    """Fixed splits put a verification's new tokens on both sides of a split boundary: each
    split's item writes its own."""
    monkeypatch.setenv("KVATTN_SPLIT_TOKENS", split)
    announce(f"append_forward across a split boundary ({split}, {dtype})")
    w = wl.make("af_boundary", seed=602, dtype=dtype, num_seqs_ctx=[2 * int(split) + 2, 1026],
                q_lens=[4, 4], num_q_heads=40, num_kv_heads=8, head_dim=128)
    a, b = DeviceCase(w), DeviceCase(w)
    a.append()
    ref = a.forward(mirror=True)
    got = b.append_forward(mirror=True)
    torch.cuda.synchronize()
    assert np.array_equal(raw(got), raw(ref))
    for x, y in zip(a.host_pools(), b.host_pools()):
        assert np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8))


@pytest.mark.parametrize("dtype,mirror", [(wl.I8, True), (wl.I8, False), (wl.BF16, True)])
def test_verification_appends_in_the_split_kernel(dtype, mirror):
    """Verification calls (1 + 3 drafts, 5 q-heads per KV head: 32-row tiles) append inside the
    split-K kernel on bf16 and int8 pools alike: no append launch, and the bits of append +
    forward.  A 16-row int8 call (decode) keeps the append kernel."""
    from paged_kv_cache_kvpool_amd import binding as kb
    announce(f"verification appends in the split kernel {dtype} mirror={mirror}")
    w = wl.make(f"af_vfuse_{dtype}", seed=604, dtype=dtype, num_seqs_ctx=[32772, 2050, 700],
                q_lens=[4, 4, 4], num_q_heads=40, num_kv_heads=8, head_dim=128)
    a, b = DeviceCase(w), DeviceCase(w)
    a.append()
    ref = a.forward(mirror=mirror)
    torch.cuda.synchronize()
    kb.kvpool_profile(True)
    got = b.append_forward(mirror=mirror)
    torch.cuda.synchronize()
    kb.kvpool_profile(False)
    launched = kb.kernel_times()
    assert "kv_append" not in launched, f"kernels {sorted(launched)}"
    assert np.array_equal(raw(got), raw(ref))
    for x, y in zip(a.host_pools(), b.host_pools()):
        assert np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8))
    # a decode call on an int8 pool (16-row tiles) appends with the append kernel
    wd = wl.make("af_vfuse_dec", seed=605, dtype=wl.I8, num_seqs_ctx=[3000, 700], q_lens=[1, 1],
                 num_q_heads=32, num_kv_heads=8, head_dim=128)
    d = DeviceCase(wd)
    kb.kvpool_profile(True)
    d.append_forward(mirror=mirror)
    torch.cuda.synchronize()
    kb.kvpool_profile(False)
    assert "kv_append" in kb.kernel_times()


def test_fp32_pool_falls_back():
    announce("append_forward fp32")
    w = wl.make("af_fp32", seed=603, dtype=wl.F32, num_seqs_ctx=[300, 700], q_lens=[1, 1],
                num_q_heads=8, num_kv_heads=8, head_dim=64)
    a, b = DeviceCase(w), DeviceCase(w)
    a.append()
    ref = a.forward(mirror=True)
    got = b.append_forward(mirror=True)
    torch.cuda.synchronize()
    assert np.array_equal(raw(got), raw(ref))


SPARSE = {  # (workload arguments, sink, window, min_len)
    "pages": (dict(num_seqs_ctx=[16383, 16384, 16385, 20000, 40000, 1000, 16400], q_lens=[1] * 7,
                   num_q_heads=32, num_kv_heads=8), 16, 4096, 16384),
    "verify": (dict(num_seqs_ctx=[16385, 16387, 16390, 30000, 16384], q_lens=[4] * 5,
                    num_q_heads=40, num_kv_heads=8), 16, 4096, 16384),
    "small": (dict(num_seqs_ctx=[700, 301, 1500, 90, 2222], q_lens=[1, 4, 2, 1, 3],
                   num_q_heads=8, num_kv_heads=2), 5, 100, 300),
}


def check_sparse(name, dtype, seed=611, mirror=True):
    cfg, sink, window, min_len = SPARSE[name]
    announce(f"append_forward_sparse {name} {dtype} mirror={mirror}")
    w = wl.make(f"afs_{name}_{dtype}", seed=seed, dtype=dtype, head_dim=128, **cfg)
    a, b = DeviceCase(w), DeviceCase(w)
    a.append()
    ref = a.forward_sparse(sink, window, min_len, mirror=mirror)
    got = b.append_forward_sparse(sink, window, min_len, mirror=mirror)
    torch.cuda.synchronize()
    assert np.array_equal(raw(got), raw(ref)), "output differs from append + forward_sparse"
    for x, y in zip(a.host_pools(), b.host_pools()):
        assert np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8)), \
            "pool differs from append + forward_sparse"
    assert_close(out_f64(got), b.oracle_sparse(sink, window, min_len), dtype, w.name, q_lens=w.q_lens)


@pytest.mark.parametrize("name", ["pages", "verify", "small"])
@pytest.mark.parametrize("dtype", [wl.BF16, wl.I8])
def test_append_forward_sparse(name, dtype):
    check_sparse(name, dtype)


def test_append_forward_sparse_without_mirror():
    check_sparse("verify", wl.BF16, mirror=False)


@pytest.mark.parametrize("split", ["256", "1024"])
def test_sparse_new_tokens_with_fixed_splits(split, monkeypatch):
    """Fixed splits cut the sparse key range (sink, then the window) into several items; the
    new tokens sit in the last one or straddle two."""
    monkeypatch.setenv("KVATTN_SPLIT_TOKENS", split)
    check_sparse("verify", wl.BF16, seed=612)
