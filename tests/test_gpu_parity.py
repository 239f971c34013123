"""GPU parity: the HIP path through the C ABI against the float64 oracle on the same seeded
inputs.  Indexing (append, block copy) is compared bit for bit over the whole pool; attention
within max-abs 2e-2 and relative L2 5e-3 for bf16, 1e-5 for fp32."""
import os
import sys

import numpy as np
import pytest
import torch

from oracle import attention as ora
from paged_kv_cache_kvpool_amd import workloads as wl

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU hosts, run on the GPU
    pytest.skip("no GPU", allow_module_level=True)

from tests.gpu_util import DeviceCase, assert_close, out_f64, to_numpy  # noqa: E402


def announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


# ---------------------------------------------------------------------------------------------
# Indexing: append and block copy, bit-exact over the whole pool
# ---------------------------------------------------------------------------------------------

APPEND_CASES = [
    dict(seed=11, dtype=wl.BF16, block_size=16, head_dim=128, num_q_heads=8, num_kv_heads=2),
    dict(seed=12, dtype=wl.BF16, block_size=64, head_dim=64, num_q_heads=4, num_kv_heads=4),
    dict(seed=13, dtype=wl.F32, block_size=16, head_dim=64, num_q_heads=2, num_kv_heads=1),
    dict(seed=14, dtype=wl.F32, block_size=64, head_dim=128, num_q_heads=6, num_kv_heads=3),
]


@pytest.mark.parametrize("kw", APPEND_CASES, ids=lambda k: f"s{k['seed']}_{k['dtype']}_B{k['block_size']}_D{k['head_dim']}")
def test_append_bitexact(kw):
    announce(f"append {kw}")
    w = wl.random_case(kw["seed"], dtype=kw["dtype"], block_size=kw["block_size"],
                       head_dim=kw["head_dim"], num_q_heads=kw["num_q_heads"],
                       num_kv_heads=kw["num_kv_heads"], num_seqs=5,
                       q_len_choices=(1, 3, 16, 17, 40), max_ctx=200)
    c = DeviceCase(w)
    c.append()
    torch.cuda.synchronize()
    k_exp, v_exp = ora.append(w.k_pool, w.v_pool, 0, w.k_new, w.v_new, w.block_tables, w.ctx_lens,
                              w.q_lens, num_kv_heads=w.num_kv_heads, block_size=w.block_size,
                              head_dim=w.head_dim, dtype=w.dtype)
    k_got, v_got = c.host_pools()
    assert k_got.tobytes() == k_exp.tobytes()
    assert v_got.tobytes() == v_exp.tobytes()


def test_append_prefix_prefill_config_bitexact():
    announce("append prefix_prefill (4 x 512 suffix rows over a 4096 prefix)")
    w = wl.prefix_prefill()
    c = DeviceCase(w)
    c.append()
    torch.cuda.synchronize()
    k_exp, v_exp = ora.append(w.k_pool, w.v_pool, 0, w.k_new, w.v_new, w.block_tables, w.ctx_lens,
                              w.q_lens, num_kv_heads=w.num_kv_heads, block_size=w.block_size,
                              head_dim=w.head_dim, dtype=w.dtype)
    k_got, v_got = c.host_pools()
    assert k_got.tobytes() == k_exp.tobytes()
    assert v_got.tobytes() == v_exp.tobytes()


def test_append_multi_layer_touches_only_its_layer():
    announce("append into layer 1 of a 3-layer pool")
    w = wl.make("layers", seed=21, dtype=wl.BF16, num_seqs_ctx=[40, 7], q_lens=[9, 7],
                num_q_heads=4, num_kv_heads=2, head_dim=64, num_layers=3, layer=1, num_blocks=8)
    c = DeviceCase(w)
    c.append()
    torch.cuda.synchronize()
    k_exp, v_exp = ora.append(w.k_pool, w.v_pool, 1, w.k_new, w.v_new, w.block_tables, w.ctx_lens,
                              w.q_lens, num_kv_heads=2, block_size=16, head_dim=64, dtype=w.dtype)
    k_got, v_got = c.host_pools()
    assert k_got.tobytes() == k_exp.tobytes() and v_got.tobytes() == v_exp.tobytes()


@pytest.mark.parametrize("dtype,block_size", [(wl.BF16, 16), (wl.F32, 64)])
def test_copy_blocks_bitexact(dtype, block_size):
    announce(f"copy_blocks {dtype} B={block_size}")
    w = wl.make("copy", seed=31, dtype=dtype, num_seqs_ctx=[100, 50], q_lens=[1, 1],
                num_q_heads=4, num_kv_heads=2, head_dim=128, num_layers=2,
                block_size=block_size, num_blocks=12, append=False)
    c = DeviceCase(w)
    src = np.array([0, 3, 7], np.int32)
    dst = np.array([5, 11, 1], np.int32)
    c.pool.copy_blocks(torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda())
    torch.cuda.synchronize()
    k_exp, v_exp = ora.copy_blocks(w.k_pool, w.v_pool, src, dst)
    k_got, v_got = c.host_pools()
    assert k_got.tobytes() == k_exp.tobytes() and v_got.tobytes() == v_exp.tobytes()


# ---------------------------------------------------------------------------------------------
# Attention parity on small ragged cases (every kernel path)
# ---------------------------------------------------------------------------------------------

SWEEP = []
for seed in range(6):
    for dtype in (wl.BF16, wl.F32):
        for (hq, hkv) in ((8, 2), (5, 1), (16, 2), (4, 4)):
            for bs in (16, 64):
                for d in (64, 128):
                    SWEEP.append((seed, dtype, hq, hkv, bs, d))
# keep the sweep to a few seconds: every combination of the small axes, a third of the seeds
SWEEP = [c for i, c in enumerate(SWEEP) if i % 3 == 0]


@pytest.mark.parametrize("seed,dtype,hq,hkv,bs,d", SWEEP,
                         ids=[f"s{c[0]}_{c[1]}_H{c[2]}x{c[3]}_B{c[4]}_D{c[5]}" for c in SWEEP])
def test_attention_random(seed, dtype, hq, hkv, bs, d):
    announce(f"random seed={seed} {dtype} Hq={hq} Hkv={hkv} B={bs} D={d}")
    w = wl.random_case(seed, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, block_size=bs,
                       head_dim=d, num_seqs=4, q_len_choices=(1, 2, 4, 17), max_ctx=300)
    c = DeviceCase(w)
    c.append()
    out = c.forward()
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle(), dtype, w.name, q_lens=w.q_lens)


@pytest.mark.parametrize("q_len", [33, 128, 200])
@pytest.mark.parametrize("dtype", [wl.BF16, wl.F32])
def test_attention_prefill_shapes(q_len, dtype):
    """Query blocks too long for split mode (prefill path), several row tiles, ragged tail."""
    announce(f"prefill shapes q_len={q_len} {dtype}")
    w = wl.make(f"prefill_{q_len}", seed=41 + q_len, dtype=dtype,
                num_seqs_ctx=[q_len + 77, q_len, q_len + 300], q_lens=[q_len, q_len, q_len // 2],
                num_q_heads=10, num_kv_heads=2, head_dim=128)
    c = DeviceCase(w)
    c.append()
    out = c.forward()
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle(), dtype, w.name, q_lens=w.q_lens)


@pytest.mark.parametrize("plan", ["4", "8", "10", "12", "12:10", "12:7", "8:5", "6:3", "5:3"])
@pytest.mark.parametrize("head_dim", [128, 64])
@pytest.mark.parametrize("dtype", [wl.BF16, wl.I8])
def test_attention_prefill_plans(plan, head_dim, dtype, monkeypatch):
    """Prefill workgroups of W waves over R row blocks (forced through KVATTN_PREFILL_WAVES and
    KVATTN_PREFILL_RBLK; "W" alone means R = W): whole-block waves only, or with pairs of half
    waves that split a row block's keys by block parity and merge at the end.  Ragged sequences
    leave partial row tiles and waves with no rows.  The plan also decides which waves stream
    the tiles (half waves, the least loaded SIMDs' waves, or all) and in which order the waves
    take the conversion units of an int8 pool, which runs here with the conversion in LDS
    (KVATTN_INT8_PREFILL=lds; with the bf16 copy the kernel is the bf16 one)."""
    if dtype == wl.I8:
        monkeypatch.setenv("KVATTN_INT8_PREFILL", "lds")
    w, _, r = plan.partition(":")
    monkeypatch.setenv("KVATTN_PREFILL_WAVES", w)
    if r:
        monkeypatch.setenv("KVATTN_PREFILL_RBLK", r)
    else:
        monkeypatch.delenv("KVATTN_PREFILL_RBLK", raising=False)
    announce(f"prefill plan {plan} D={head_dim} {dtype}")
    w = wl.make(f"prefill_plan_{plan.replace(':', 'r')}_{head_dim}_{dtype}", seed=61, dtype=dtype,
                num_seqs_ctx=[700, 450, 130, 1300], q_lens=[300, 450, 97, 64],
                num_q_heads=10, num_kv_heads=2, head_dim=head_dim)
    c = DeviceCase(w)
    c.append()
    out = c.forward()
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle(), dtype, w.name, q_lens=w.q_lens)


MIXED_CASES = [
    # (dtype, Hq, Hkv, D, B): G = 4, 5, 8 and 1; both head dims and block sizes
    (wl.BF16, 32, 8, 128, 16),
    (wl.BF16, 40, 8, 128, 64),
    (wl.BF16, 16, 2, 64, 16),
    (wl.BF16, 4, 4, 64, 64),
    (wl.F32, 10, 2, 64, 16),
]


@pytest.mark.parametrize("mirror", [False, True], ids=["bounds", "mirror"])
@pytest.mark.parametrize("dtype,hq,hkv,d,bs", MIXED_CASES,
                         ids=[f"{c[0]}_H{c[1]}x{c[2]}_D{c[3]}_B{c[4]}" for c in MIXED_CASES])
def test_mixed_step(dtype, hq, hkv, d, bs, mirror):
    """Decode, verification and prefill sequences in one call: each takes the kernel its own
    q_len selects (split-K up to 128 rows per KV head, the prefill kernel past that), with
    empty and one-key sequences between them; grids sized from the bounds, or exactly from the
    host mirror of q_lens."""
    announce(f"mixed step {dtype} Hq={hq} Hkv={hkv} D={d} B={bs} mirror={mirror}")
    w = wl.make(f"mixed_{dtype}_{hq}_{d}_{bs}", seed=141 + hq + d + bs, dtype=dtype,
                num_seqs_ctx=[3000, 700, 1000, 1, 129, 9000, 50, 300, 20],
                q_lens=[1, 4, 300, 1, 129, 4, 0, 33, 20],
                num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs)
    c = DeviceCase(w)
    c.append()
    out = c.forward(mirror=mirror)
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle(), dtype, w.name, q_lens=w.q_lens)


def test_decode_vec_kernel_bf16(monkeypatch):
    """The vector-ALU bf16 decode variant (selected by KVATTN_DECODE_VEC=1)."""
    monkeypatch.setenv("KVATTN_DECODE_VEC", "1")
    announce("bf16 decode on the vector-ALU kernel")
    w = wl.make("vec_decode", seed=51, dtype=wl.BF16, num_seqs_ctx=[1000, 17, 4096, 1],
                q_lens=[1, 1, 1, 1], num_q_heads=32, num_kv_heads=8, head_dim=128)
    c = DeviceCase(w)
    c.append()
    out = c.forward()
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle(), wl.BF16, w.name, q_lens=w.q_lens)


@pytest.mark.parametrize("dtype,head_dim", [(wl.F32, 64), (wl.F32, 128), (wl.BF16, 128), (wl.BF16, 64)])
def test_decode_vec_single_row_waves(dtype, head_dim, monkeypatch):
    """One q-head per KV head (single-row waves: four waves share each split and merge in
    LDS): contexts from 1 key (three waves without a tile) through 17 and 300 keys to several
    splits (their partials merged by the reduce); bf16 through KVATTN_DECODE_VEC=1."""
    if dtype == wl.BF16:
        monkeypatch.setenv("KVATTN_DECODE_VEC", "1")
    announce(f"single-row vec decode {dtype} d={head_dim}")
    w = wl.make(f"vec_rows1_{dtype}_{head_dim}", seed=52, dtype=dtype,
                num_seqs_ctx=[1, 17, 300, 513, 1030, 5000, 64, 2049], q_lens=[1] * 8,
                num_q_heads=8, num_kv_heads=8, head_dim=head_dim)
    c = DeviceCase(w)
    c.append()
    for mirror in (False, True):
        out = c.forward(mirror=mirror)
        torch.cuda.synchronize()
        assert_close(out_f64(out), c.oracle(), dtype, w.name, q_lens=w.q_lens)


# ---------------------------------------------------------------------------------------------
# The five measured workloads at full size
# ---------------------------------------------------------------------------------------------

def test_tiny_decode_fp32():
    announce("tiny_decode fp32 (1 seq, 256 keys in 16 of 32 blocks, D=64)")
    w = wl.tiny_decode()
    c = DeviceCase(w)
    out = c.forward()
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle(), wl.F32, w.name, q_lens=w.q_lens)


def test_batched_gqa_decode_full():
    announce("batched_gqa_decode (32 seqs, 1024..8192 keys, 32/8 heads)")
    w = wl.batched_gqa_decode()
    c = DeviceCase(w)
    c.append()
    out = c.forward()
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle(), wl.BF16, w.name, q_lens=w.q_lens)


@pytest.mark.parametrize("cached", [32768, 131072])
def test_spec_verify_full(cached):
    announce(f"spec_verify cached={cached} (1 seq, 1+3 tokens, 40/8 heads)")
    w = wl.spec_verify(cached=cached)
    c = DeviceCase(w)
    c.append()
    out = c.forward()
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle(), wl.BF16, w.name, q_lens=w.q_lens)


def test_prefix_prefill_full():
    announce("prefix_prefill (4 x (4096 cached + 512 new), 40/8 heads)")
    w = wl.prefix_prefill()
    c = DeviceCase(w)
    c.append()
    out = c.forward()
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle(), wl.BF16, w.name, q_lens=w.q_lens)


def test_mixed_step_full():
    announce("mixed_step (32 decode + 1 verify at 32768 + 1 prefill chunk of 512 over 4096)")
    w = wl.mixed_step()
    c = DeviceCase(w)
    c.append()
    out = c.forward(mirror=True)
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle(), wl.BF16, w.name, q_lens=w.q_lens)


def test_long_decode_full():
    announce("long_decode (262144 + 131072 keys, pool of 24576 blocks drawn on the device)")
    w = wl.long_decode()
    c = DeviceCase(w)
    kh, vh = c.host_pools()
    c.append()
    out = c.forward()
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle(kh, vh), wl.BF16, w.name, q_lens=w.q_lens)
