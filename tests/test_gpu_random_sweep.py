"""Seeded random sweep over the call space (beside the hand-picked cases): each case draws a
batch of sequences whose query lengths mix decode (1), verification (2..8) and prefill chunks
(17..300), contexts from 1 to 3000 keys, GQA ratios 1..8, head dims 64 and 128, block sizes 16
and 64 and the three pool types, and runs it as kvpool_append + kvattn_forward and as
kvattn_append_forward (with and without the host mirror of q_lens).  The two must give the same
output and pool bits, and the output must match the oracle (the pages' attention over the
block-paged pool: sparkinfer server README, "Request isolation & continuous batching",
"Automatic prefix cache").  A second sweep does the same for sink + window sparse calls
(decode and verification rows; random sink, window and threshold: sparkinfer server README,
"Env", SPARKINFER_SPARSE_GQA6).  Inputs are drawn from the seed alone; nothing here is stored.
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

N_CASES = 150
N_SPARSE = 60


def announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def raw(t):
    return t.detach().contiguous().view(torch.uint8).cpu().numpy()


def draw_case(seed):
    rng = np.random.default_rng(10_000 + seed)
    dtype = [wl.BF16, wl.I8, wl.F32][seed % 3]
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 5, 8]))
    d = int(rng.choice([64, 128]))
    bs = int(rng.choice([16, 64]))
    n = int(rng.integers(1, 9))
    kinds = rng.choice(["decode", "verify", "prefill"], size=n, p=[0.5, 0.3, 0.2])
    ctx, ql = [], []
    for k in kinds:
        q = (1 if k == "decode" else int(rng.integers(2, 9)) if k == "verify"
             else int(rng.integers(17, 301)))
        c = int(rng.integers(q, 3001))
        ctx.append(c)
        ql.append(q)
    return dict(dtype=dtype, num_seqs_ctx=ctx, q_lens=ql, num_q_heads=hkv * g, num_kv_heads=hkv,
                head_dim=d, block_size=bs)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_batch(seed):
    cfg = draw_case(seed)
    dtype = cfg.pop("dtype")
    mirror = bool(seed % 2)
    announce(f"random batch {seed}: {dtype} ctx={cfg['num_seqs_ctx']} q={cfg['q_lens']} "
             f"heads={cfg['num_q_heads']}/{cfg['num_kv_heads']} d={cfg['head_dim']} "
             f"bs={cfg['block_size']} mirror={mirror}")
    w = wl.make(f"sweep_{seed}", seed=20_000 + seed, dtype=dtype, **cfg)
    a, b = DeviceCase(w), DeviceCase(w)
    a.append()
    ref = a.forward(mirror=mirror)
    got = b.append_forward(mirror=mirror)
    torch.cuda.synchronize()
    assert np.array_equal(raw(got), raw(ref)), "append_forward output differs from append + forward"
    for x, y in zip(a.host_pools(), b.host_pools()):
        assert np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8)), \
            "append_forward pool differs from append + forward"
    assert_close(out_f64(got), b.oracle(), dtype, w.name, q_lens=w.q_lens)


def draw_sparse(seed):
    rng = np.random.default_rng(30_000 + seed)
    dtype = [wl.BF16, wl.I8][seed % 2]
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 5, 8]))
    n = int(rng.integers(1, 9))
    ql = [1 if rng.random() < 0.6 else int(rng.integers(2, 9)) for _ in range(n)]
    ctx = [int(rng.integers(q, 3001)) for q in ql]
    sparse = (int(rng.choice([0, 3, 16, 40])), int(rng.choice([1, 33, 200, 700])),
              int(rng.choice([0, 100, 1500])))
    cfg = dict(num_seqs_ctx=ctx, q_lens=ql, num_q_heads=hkv * g, num_kv_heads=hkv,
               head_dim=int(rng.choice([64, 128])), block_size=int(rng.choice([16, 64])))
    return dtype, cfg, sparse


@pytest.mark.parametrize("seed", range(N_SPARSE))
def test_random_sparse_batch(seed):
    dtype, cfg, (sink, window, min_len) = draw_sparse(seed)
    mirror = bool(seed % 3)
    announce(f"random sparse batch {seed}: {dtype} ctx={cfg['num_seqs_ctx']} q={cfg['q_lens']} "
             f"heads={cfg['num_q_heads']}/{cfg['num_kv_heads']} d={cfg['head_dim']} "
             f"bs={cfg['block_size']} sink={sink} window={window} min={min_len} mirror={mirror}")
    w = wl.make(f"sweep_sp_{seed}", seed=40_000 + seed, dtype=dtype, **cfg)
    a, b = DeviceCase(w), DeviceCase(w)
    a.append()
    ref = a.forward_sparse(sink, window, min_len, mirror=mirror)
    got = b.append_forward_sparse(sink, window, min_len, mirror=mirror)
    torch.cuda.synchronize()
    assert np.array_equal(raw(got), raw(ref)), \
        "append_forward_sparse differs from append + forward_sparse"
    for x, y in zip(a.host_pools(), b.host_pools()):
        assert np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8))
    assert_close(out_f64(got), b.oracle_sparse(sink, window, min_len), dtype, w.name,
                 q_lens=w.q_lens)
