"""GPU parity with more sequences than one wave's 64 lanes: the kernels find a work item's
sequence by scanning the sequences 64 at a time (split-K items, partial rows of the reduce,
prefill tiles, the first row of each sequence), and these calls cross several such groups.
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


def bits(t):
    return t.detach().view(torch.int16).cpu().numpy()


def many(seed, n, dtype, q_choices, max_ctx, hq=16, hkv=4, d=128):
    rng = np.random.default_rng(seed)
    ql = rng.choice(np.asarray(q_choices), size=n).astype(np.int32)
    ctx = np.array([int(rng.integers(int(t), max(int(t), max_ctx) + 1)) for t in ql], np.int32)
    return wl.make(f"many_{n}_{dtype}", seed=seed, dtype=dtype, num_seqs_ctx=ctx, q_lens=ql,
                   num_q_heads=hq, num_kv_heads=hkv, head_dim=d)


@pytest.mark.parametrize("dtype", [wl.BF16, wl.I8])
def test_many_sequences_decode(dtype):
    announce(f"200-sequence decode {dtype}")
    w = many(401, 200, dtype, (1,), 3000)
    c = DeviceCase(w)
    c.append()
    out = c.forward()
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle(), dtype, w.name, q_lens=w.q_lens)


@pytest.mark.parametrize("mirror", [False, True], ids=["bounds", "mirror"])
def test_many_sequences_mixed(mirror):
    """150 sequences of decode (q_len 1), verification (4) and prefill chunks (40 and 200 rows
    x 4 q-heads per KV head) in one call."""
    announce(f"150-sequence mixed call mirror={mirror}")
    w = many(402, 150, wl.BF16, (1, 1, 1, 4, 40, 200), 1500)
    c = DeviceCase(w)
    c.append()
    out = c.forward(mirror=mirror)
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle(), wl.BF16, w.name, q_lens=w.q_lens)


def test_many_sequences_sparse():
    announce("70-sequence sparse decode")
    rng = np.random.default_rng(403)
    ctx = rng.integers(1, 2600, size=70).astype(np.int32)
    w = wl.make("many_sparse", seed=403, dtype=wl.BF16, num_seqs_ctx=ctx,
                q_lens=np.where(np.arange(70) % 5 == 0, np.minimum(ctx, 4), 1).astype(np.int32),
                num_q_heads=16, num_kv_heads=4, head_dim=128)
    c = DeviceCase(w)
    c.append()
    out = c.forward_sparse(16, 500, 1000)
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle_sparse(16, 500, 1000), wl.BF16, w.name, q_lens=w.q_lens)


def test_many_sequences_batch_invariance(monkeypatch):
    """In deterministic mode, sequences in the second and third group of 64 give the same bits
    alone as in the batch (prefill-class ones included)."""
    monkeypatch.setenv("KVATTN_DETERMINISTIC", "1")
    announce("batch invariance past 64 sequences")
    w = many(404, 160, wl.BF16, (1, 1, 4, 200), 2000)
    c = DeviceCase(w)
    c.append()
    full = c.forward()
    torch.cuda.synchronize()
    starts = np.concatenate([[0], np.cumsum(w.q_lens)])
    for s in (0, 63, 64, 65, 127, 128, 159):
        rows = slice(int(starts[s]), int(starts[s + 1]))
        sel = torch.tensor([s], device="cuda")
        alone = c.pool.forward(0, c.q[rows], c.tables[sel], c.ctx[sel], c.ql[sel], scale=w.scale,
                               max_ctx_len=int(w.ctx_lens[s]), max_q_len=int(w.q_lens[s]))
        torch.cuda.synchronize()
        assert np.array_equal(bits(alone), bits(full[rows])), f"sequence {s}"


@pytest.mark.parametrize("plan", ["8:4", "12:10", "10:5", "6:3", "12"])
def test_prefill_short_prefix_half_pairs(plan, monkeypatch):
    """Prefill chunks over prefixes shorter than one 32-key block, under plans with half-wave
    pairs: a row block then straddles a block boundary, so the odd wave of a pair holds rows
    none of whose keys are in its blocks (they must contribute nothing, not NaN)."""
    w_, _, r_ = plan.partition(":")
    monkeypatch.setenv("KVATTN_PREFILL_WAVES", w_)
    if r_:
        monkeypatch.setenv("KVATTN_PREFILL_RBLK", r_)
    else:
        monkeypatch.delenv("KVATTN_PREFILL_RBLK", raising=False)
    announce(f"short-prefix prefill under plan {plan}")
    w = wl.make(f"short_prefix_{plan.replace(':', 'r')}", seed=405, dtype=wl.BF16,
                num_seqs_ctx=[223, 218, 240, 40, 231, 300], q_lens=[200, 200, 210, 33, 231, 290],
                num_q_heads=16, num_kv_heads=4, head_dim=128)
    c = DeviceCase(w)
    c.append()
    out = c.forward(mirror=True)
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle(), wl.BF16, w.name, q_lens=w.q_lens)
