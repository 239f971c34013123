"""GPU parity of the int8 KV pool through the C ABI.

The append quantises bf16 rows into codes and per-(token, KV head) scales and is compared bit
for bit (codes and scales, whole pool) with the oracle's quantising append; block copy moves
codes and scales bit for bit.  Attention on an int8 pool is compared with the oracle run on the
exactly dequantized K/V, at the bf16 bar (max-abs 2e-2, relative L2 5e-3): decode and
verification read the codes directly; prefill reads a bf16 copy dequantized into the workspace
when the workspace holds it, else converts the codes to bf16 in its LDS stages.  Either way it
must give, bit for bit, the prefill kernel's output on a bf16 pool holding bf16(f32(code *
scale)) of every element (test_int8_prefill_equals_bf16_of_dequantized).

The pages report a GQA-fused int8 prefill attention whose results break down from 2048 prompt
tokens up (sparkinfer server README, "Determinism", known defect); test_int8_prefill_lengths
runs whole prompts of 1500 to 4000 tokens through the GQA-fused prefill kernel on an int8 pool.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

from oracle import brute
from oracle import quant as oq
from paged_kv_cache_kvpool_amd import workloads as wl

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from paged_kv_cache_kvpool_amd import binding as kb  # noqa: E402
from tests.gpu_util import DeviceCase, assert_close, out_f64  # noqa: E402


def announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def bits(t):
    return t.detach().view(torch.int16).cpu().numpy()


@pytest.mark.parametrize("bs,d,hkv", [(16, 128, 2), (64, 64, 4), (16, 64, 1), (64, 128, 3)])
def test_append_int8_bitexact(bs, d, hkv):
    announce(f"int8 append B={bs} D={d} Hkv={hkv}")
    w = wl.random_case(20 + bs + d + hkv, dtype=wl.I8, block_size=bs, head_dim=d,
                       num_q_heads=2 * hkv, num_kv_heads=hkv, num_seqs=5,
                       q_len_choices=(1, 3, 16, 17, 40), max_ctx=200)
    c = DeviceCase(w)
    c.append()
    torch.cuda.synchronize()
    kp, vp, ks, vs = oq.append(w.k_pool, w.v_pool, w.k_scales, w.v_scales, 0, w.k_new, w.v_new,
                               w.block_tables, w.ctx_lens, w.q_lens, num_kv_heads=hkv,
                               block_size=bs, head_dim=d)
    gk, gv, gks, gvs = c.host_pools()
    assert np.array_equal(gk, kp) and np.array_equal(gv, vp)
    # scales: compare bits (unreferenced blocks hold NaN canaries on both sides)
    assert np.array_equal(gks.view(np.uint32), ks.view(np.uint32))
    assert np.array_equal(gvs.view(np.uint32), vs.view(np.uint32))


def test_copy_blocks_int8_bitexact():
    announce("int8 copy_blocks")
    w = wl.make("copy_i8", seed=31, dtype=wl.I8, num_seqs_ctx=[100, 50], q_lens=[1, 1],
                num_q_heads=4, num_kv_heads=2, head_dim=128, num_layers=2, num_blocks=12,
                append=False)
    c = DeviceCase(w)
    src = np.array([0, 3, 7], np.int32)
    dst = np.array([5, 11, 1], np.int32)
    c.pool.copy_blocks(torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda())
    torch.cuda.synchronize()
    kp, vp, ks, vs = oq.copy_blocks(w.k_pool, w.v_pool, w.k_scales, w.v_scales, src, dst)
    gk, gv, gks, gvs = c.host_pools()
    assert np.array_equal(gk, kp) and np.array_equal(gv, vp)
    assert np.array_equal(gks.view(np.uint32), ks.view(np.uint32))
    assert np.array_equal(gvs.view(np.uint32), vs.view(np.uint32))


SWEEP = [(seed, hq, hkv, bs, d) for seed in range(3) for (hq, hkv) in ((8, 2), (5, 1), (16, 2), (4, 4))
         for bs in (16, 64) for d in (64, 128)]
SWEEP = [c for i, c in enumerate(SWEEP) if i % 3 == 0]


@pytest.mark.parametrize("seed,hq,hkv,bs,d", SWEEP,
                         ids=[f"s{c[0]}_H{c[1]}x{c[2]}_B{c[3]}_D{c[4]}" for c in SWEEP])
def test_attention_int8_random(seed, hq, hkv, bs, d):
    announce(f"int8 random seed={seed} Hq={hq} Hkv={hkv} B={bs} D={d}")
    w = wl.random_case(seed, dtype=wl.I8, num_q_heads=hq, num_kv_heads=hkv, block_size=bs,
                       head_dim=d, num_seqs=4, q_len_choices=(1, 2, 4, 17), max_ctx=300)
    c = DeviceCase(w)
    c.append()
    out = c.forward()
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle(), wl.I8, w.name, q_lens=w.q_lens)


@pytest.mark.parametrize("prompt", [1500, 2000, 2047, 2048, 2049, 2100, 3000, 4000])
def test_int8_prefill_lengths(prompt):
    """A whole prompt prefilled at once over an int8 pool, GQA-fused (4 q-heads per KV head):
    every row against the oracle, on both sides of 2048 tokens."""
    announce(f"int8 prefill prompt={prompt}")
    w = wl.make(f"i8_prompt_{prompt}", seed=prompt, dtype=wl.I8, num_seqs_ctx=[prompt],
                q_lens=[prompt], num_q_heads=4, num_kv_heads=1, head_dim=64)
    c = DeviceCase(w)
    c.append()
    out = c.forward(mirror=True)
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle(), wl.I8, w.name, q_lens=w.q_lens)


def bf16_pool_of_dequantized(w, k8, v8, ks, vs):
    """Raw bf16 K/V storage (8-dim K chunks) holding, for every element of the int8 pool
    (k8, v8: raw codes; ks, vs: scales [layers][blocks][Hkv][B]), the nearest-even bf16 of the
    float32 product code * scale; placed with the storage offset formulas of oracle.brute."""
    geo = dict(num_kv_heads=w.num_kv_heads, block_size=w.block_size, head_dim=w.head_dim)
    b, h, t, d = np.meshgrid(np.arange(w.num_blocks), np.arange(w.num_kv_heads),
                             np.arange(w.block_size), np.arange(w.head_dim), indexing="ij")
    src = (brute.k_offset_i8(b, h, t, d, **geo), brute.v_offset_i8(b, h, t, d, **geo))
    dst = (brute.k_offset(b, h, t, d, x=8, **geo), brute.v_offset(b, h, t, d, **geo))
    out = []
    for raw, sc, si, di in ((k8, ks, src[0], dst[0]), (v8, vs, src[1], dst[1])):
        pool = np.empty((w.num_layers, w.num_blocks * w.block_elems), dtype=np.uint16)
        for layer in range(w.num_layers):
            codes = raw[layer].reshape(-1).view(np.int8)[si].astype(np.float32)
            with np.errstate(invalid="ignore"):  # NaN canary scales of unreferenced blocks
                val = codes * sc[layer][b, h, t].astype(np.float32)  # one float32 rounding
            pool[layer][di.reshape(-1)] = wl.rne_bf16_bits(val).reshape(-1)
        out.append(pool.reshape(w.num_layers, w.num_blocks, w.block_elems))
    return out


@pytest.mark.parametrize("path", ["copy", "lds"])
@pytest.mark.parametrize("hq,hkv,d,bs,ctx,ql", [
    (40, 8, 128, 16, [700, 1100, 333], [300, 64, 333]),
    (16, 2, 64, 64, [2100, 517], [129, 517]),
    (8, 1, 128, 64, [4097], [200]),
    (4, 1, 64, 16, [1500], [1500]),
], ids=["H40x8_D128_B16", "H16x2_D64_B64", "H8x1_D128_B64_long", "H4x1_D64_prompt"])
def test_int8_prefill_equals_bf16_of_dequantized(hq, hkv, d, bs, ctx, ql, path, monkeypatch):
    """Both int8 prefill paths turn each code into bf16(f32(code * scale)) (keys past the
    context zero) before the bf16 prefill arithmetic: "copy" into a workspace pool that the bf16
    kernel reads, "lds" (KVATTN_INT8_PREFILL=lds, the path taken when the workspace has no room
    for the copy) inside the kernel's LDS stages.  So the output equals, bit for bit, the bf16
    kernel's on a bf16 pool holding those values (same rows, same plan: every sequence
    prefill-class).  Exercises ragged last tiles, both head dims and block sizes, key ranges (few
    workgroups) and whole prompts."""
    if path == "lds":
        monkeypatch.setenv("KVATTN_INT8_PREFILL", "lds")
    else:
        monkeypatch.delenv("KVATTN_INT8_PREFILL", raising=False)
    announce(f"int8 prefill ({path}) == bf16 of dequantized Hq={hq} Hkv={hkv} D={d} B={bs} "
             f"ctx={ctx} q={ql}")
    w = wl.make(f"i8_eq_{hq}_{d}_{bs}", seed=191 + hq + d + bs + len(ctx), dtype=wl.I8,
                num_seqs_ctx=ctx, q_lens=ql, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                block_size=bs)
    assert all(q * (hq // hkv) > 128 for q in ql)  # prefill-class (more than 128 rows per KV head)
    c = DeviceCase(w)
    c.append()
    out8 = c.forward(mirror=True)
    torch.cuda.synchronize()
    kb, vb = bf16_pool_of_dequantized(w, *c.host_pools())
    wb = dataclasses.replace(w, name=w.name + "_bf16", dtype=wl.BF16, k_pool=kb, v_pool=vb,
                             k_scales=None, v_scales=None, k_new=None, v_new=None)
    monkeypatch.delenv("KVATTN_INT8_PREFILL", raising=False)
    cb = DeviceCase(wb)
    outb = cb.forward(mirror=True)
    torch.cuda.synchronize()
    a, r = bits(out8), bits(outb)
    print(f"[parity] {w.name}: {int(np.count_nonzero(a != r))} of {a.size} outputs differ", flush=True)
    assert np.array_equal(a, r)
    assert_close(out_f64(out8), c.oracle(), wl.I8, w.name, q_lens=w.q_lens)


def test_int8_prefill_short_workspace_takes_lds_path():
    """A workspace smaller than kvattn_workspace_size asks (which counts the bf16 copy) but
    large enough for the rest: the call runs, converting in LDS, with the same bits as with
    the full workspace (mixed call: decode, verification and prefill rows)."""
    announce("int8 prefill with a workspace short of the bf16 copy")
    w = wl.make("i8_short_ws", seed=197, dtype=wl.I8, num_seqs_ctx=[3000, 700, 1000, 2600],
                q_lens=[1, 4, 300, 129], num_q_heads=40, num_kv_heads=8, head_dim=128)
    c = DeviceCase(w)
    c.append()
    full = c.forward(mirror=True)
    need = kb.kvattn_workspace_size(c.pool.handle, w.num_q_heads, w.num_seqs, w.total_q,
                                    int(w.ctx_lens.max()), int(w.q_lens.max()), w.q_lens)
    short = need - 256  # no room for the copy (it holds at least 2 x 700 x 16 x D bytes)
    ws = torch.empty(short, dtype=torch.uint8, device="cuda")
    out = torch.full_like(c.q, float("nan"))
    kb.kvattn_forward(c.pool.handle, w.layer, c.q, out, w.num_q_heads, w.scale, c.tables,
                      c.tables.shape[1], c.ctx, c.ql, w.num_seqs, w.total_q,
                      int(w.ctx_lens.max()), int(w.q_lens.max()), ws, short, q_lens_host=w.q_lens)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), bits(full))
    assert_close(out_f64(out), c.oracle(), wl.I8, w.name, q_lens=w.q_lens)


@pytest.mark.parametrize("mirror", [False, True], ids=["bounds", "mirror"])
@pytest.mark.parametrize("hq,hkv,d,bs", [(32, 8, 128, 16), (40, 8, 128, 64), (16, 2, 64, 16)])
def test_mixed_step_int8(hq, hkv, d, bs, mirror):
    announce(f"int8 mixed step Hq={hq} Hkv={hkv} D={d} B={bs} mirror={mirror}")
    w = wl.make(f"i8_mixed_{hq}_{d}_{bs}", seed=171 + hq + d + bs, dtype=wl.I8,
                num_seqs_ctx=[3000, 700, 1000, 1, 129, 9000, 50, 300, 20],
                q_lens=[1, 4, 300, 1, 129, 4, 0, 33, 20],
                num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs)
    c = DeviceCase(w)
    c.append()
    out = c.forward(mirror=mirror)
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle(), wl.I8, w.name, q_lens=w.q_lens)


def test_int8_batch_invariance_bitwise(monkeypatch):
    """On an int8 pool too, in deterministic mode, each sequence of a mixed call gives alone the
    same bits."""
    monkeypatch.setenv("KVATTN_DETERMINISTIC", "1")
    announce("int8 mixed batch invariance")
    w = wl.make("i8_inv", seed=181, dtype=wl.I8, num_seqs_ctx=[3000, 700, 1000, 9000, 129, 40],
                q_lens=[1, 4, 300, 4, 129, 33], num_q_heads=40, num_kv_heads=8, head_dim=128)
    c = DeviceCase(w)
    c.append()
    full = c.forward()
    again = c.forward(mirror=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits(full), bits(again))
    starts = np.concatenate([[0], np.cumsum(w.q_lens)])
    for s in range(w.num_seqs):
        rows = slice(int(starts[s]), int(starts[s + 1]))
        sel = torch.tensor([s], device="cuda")
        alone = c.pool.forward(0, c.q[rows], c.tables[sel], c.ctx[sel], c.ql[sel], scale=w.scale,
                               max_ctx_len=int(w.ctx_lens[s]), max_q_len=int(w.q_lens[s]))
        torch.cuda.synchronize()
        assert np.array_equal(bits(alone), bits(full[rows])), f"sequence {s}"


# ---- the measured workloads on int8 pools, full size ---------------------------------------------

def test_batched_gqa_decode_int8_full():
    announce("batched_gqa_decode_int8")
    w = wl.batched_gqa_decode(dtype=wl.I8)
    c = DeviceCase(w)
    c.append()
    out = c.forward(mirror=True)
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle(), wl.I8, w.name, q_lens=w.q_lens)


@pytest.mark.parametrize("cached", [32768, 131072])
def test_spec_verify_int8_full(cached):
    announce(f"spec_verify_int8 cached={cached}")
    w = wl.spec_verify(cached=cached, dtype=wl.I8)
    c = DeviceCase(w)
    c.append()
    out = c.forward(mirror=True)
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle(), wl.I8, w.name, q_lens=w.q_lens)


def test_prefix_prefill_int8_full():
    announce("prefix_prefill_int8")
    w = wl.prefix_prefill(dtype=wl.I8)
    c = DeviceCase(w)
    c.append()
    out = c.forward(mirror=True)
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle(), wl.I8, w.name, q_lens=w.q_lens)


def test_long_decode_int8_full():
    announce("long_decode_int8 (pool drawn on the device)")
    w = wl.long_decode(dtype=wl.I8)
    c = DeviceCase(w)
    kh, vh, ksh, vsh = c.host_pools()
    c.append()
    out = c.forward(mirror=True)
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle(kh, vh, scales=(ksh, vsh)), wl.I8, w.name)


def test_mixed_step_int8_full():
    announce("mixed_step_int8")
    w = wl.mixed_step(dtype=wl.I8)
    c = DeviceCase(w)
    c.append()
    out = c.forward(mirror=True)
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle(), wl.I8, w.name, q_lens=w.q_lens)
