"""GPU invariants and edge cases of the HIP path (through the C ABI), beside the oracle parity:

* physical block placement, batch composition and repetition change no output bit;
* slots past ctx_len and blocks no table reaches may hold NaN;
* verification row i equals a decode step at its own length; suffix-only prefill over a cached
  prefix equals the last rows of a one-pass prefill (both within the bf16 tolerance);
* host-side validation answers bad metadata with the documented error codes;
* ragged and degenerate shapes (q_len 0, one key, contexts shorter than a block, every GQA
  ratio up to 16, forced split sizes that exercise every kernel variant).
"""
import sys

import numpy as np
import pytest
import torch

from oracle import attention as ora
from paged_kv_cache_kvpool_amd import workloads as wl

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from paged_kv_cache_kvpool_amd import binding as kb  # noqa: E402
from tests.gpu_util import DeviceCase, assert_close, out_f64, to_torch  # noqa: E402


def announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def bits(t):
    return t.detach().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


MIXED = dict(seed=61, dtype=wl.BF16, num_seqs_ctx=[3000, 700, 40, 9000], q_lens=[1, 4, 1, 4],
             num_q_heads=40, num_kv_heads=8, head_dim=128)


def test_placement_invariance_bitwise():
    announce("placement invariance (decode + verify rows)")
    w = wl.make("placement", **MIXED)
    c1 = DeviceCase(w)
    c1.append()
    o1 = c1.forward()
    # same logical data, every block moved to another physical id
    perm = np.random.default_rng(7).permutation(w.num_blocks).astype(np.int32)
    w2 = wl.make("placement", **MIXED)
    w2.k_pool = np.empty_like(w.k_pool)
    w2.v_pool = np.empty_like(w.v_pool)
    w2.k_pool[:, perm] = w.k_pool
    w2.v_pool[:, perm] = w.v_pool
    w2.block_tables = perm[w.block_tables]
    c2 = DeviceCase(w2)
    c2.append()
    o2 = c2.forward()
    torch.cuda.synchronize()
    assert np.array_equal(bits(o1), bits(o2))


@pytest.mark.parametrize("dtype", [wl.BF16, wl.F32])
def test_batch_invariance_and_repeatability_bitwise(dtype):
    announce(f"batch invariance {dtype}")
    kw = dict(MIXED, dtype=dtype)
    w = wl.make("batch", **kw)
    c = DeviceCase(w)
    c.append()
    full = c.forward()
    again = c.forward()
    torch.cuda.synchronize()
    assert np.array_equal(bits(full), bits(again)), "run-to-run"
    starts = np.concatenate([[0], np.cumsum(w.q_lens)])
    for s in range(w.num_seqs):
        rows = slice(int(starts[s]), int(starts[s + 1]))
        sel = torch.tensor([s], device="cuda")
        alone = c.pool.forward(0, c.q[rows], c.tables[sel], c.ctx[sel], c.ql[sel], scale=w.scale,
                               max_ctx_len=int(w.ctx_lens.max()), max_q_len=int(w.q_lens.max()))
        torch.cuda.synchronize()
        assert np.array_equal(bits(alone), bits(full[rows])), f"sequence {s}"


@pytest.mark.parametrize("dtype", [wl.BF16, wl.F32])
def test_mixed_batch_invariance_bitwise(dtype, monkeypatch):
    """In deterministic mode (KVATTN_DETERMINISTIC=1, as the pages' servers offer bit-reproducible,
    batch-invariant output as a mode: sparkinfer server README, "Determinism"), decode,
    verification and prefill sequences in one call give, bit for bit, what each gives alone with
    bounds of its own (max_ctx_len, max_q_len): the kernel and the split plan follow from the
    sequence itself, and prefill row blocks are always reduced by one wave in key order."""
    monkeypatch.setenv("KVATTN_DETERMINISTIC", "1")
    announce(f"mixed batch invariance {dtype}")
    w = wl.make("mixed_inv", seed=151, dtype=dtype, num_seqs_ctx=[3000, 700, 1000, 9000, 129, 40],
                q_lens=[1, 4, 300, 4, 129, 33], num_q_heads=40, num_kv_heads=8, head_dim=128)
    c = DeviceCase(w)
    c.append()
    full = c.forward()
    exact = c.forward(mirror=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits(full), bits(exact)), "bounds vs host mirror"
    starts = np.concatenate([[0], np.cumsum(w.q_lens)])
    for s in range(w.num_seqs):
        rows = slice(int(starts[s]), int(starts[s + 1]))
        sel = torch.tensor([s], device="cuda")
        for mirror in (None, w.q_lens[s:s + 1]):
            alone = c.pool.forward(0, c.q[rows], c.tables[sel], c.ctx[sel], c.ql[sel],
                                   scale=w.scale, max_ctx_len=int(w.ctx_lens[s]),
                                   max_q_len=int(w.q_lens[s]), q_lens_host=mirror)
            torch.cuda.synchronize()
            assert np.array_equal(bits(alone), bits(full[rows])), f"sequence {s} mirror={mirror}"


@pytest.mark.parametrize("dtype", [wl.BF16, wl.I8])
def test_decode_beside_verification_two_launches(dtype):
    """Decode sequences (5 rows per KV head) beside verifications (20 rows) in one call: with the
    host's q_lens the decode sequences take the 16-row kernel and the verifications the 32-row
    one (two launches); from the bounds alone, one 32-row launch serves all.  Both plans give
    the same bits (a row's arithmetic does not depend on the tile it shares), and they match
    the oracle."""
    announce(f"decode beside verification, two launches, {dtype}")
    w = wl.make(f"two_launch_{dtype}", seed=152, dtype=dtype,
                num_seqs_ctx=[3000, 32772, 700, 9000, 5000, 2050, 17, 4100],
                q_lens=[1, 4, 1, 1, 4, 4, 1, 1], num_q_heads=40, num_kv_heads=8, head_dim=128)
    c = DeviceCase(w)
    c.append()
    one = c.forward()
    two = c.forward(mirror=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits(one), bits(two)), "one launch vs two"
    assert_close(out_f64(two), c.oracle(), dtype, w.name, q_lens=w.q_lens)


@pytest.mark.parametrize("dtype", [wl.BF16, wl.I8, wl.F32])
@pytest.mark.parametrize("mirror", [False, True], ids=["bounds", "mirror"])
def test_short_decode_without_reduce(dtype, mirror):
    """Decode sequences of at most 512 keys (single-tile rows take 512-key splits): the call
    skips the reduce launch, and every row still matches the oracle."""
    announce(f"short decode without reduce {dtype} mirror={mirror}")
    w = wl.make(f"short_dec_{dtype}", seed=153, dtype=dtype,
                num_seqs_ctx=[300, 400, 512, 257, 511, 33], q_lens=[1] * 6, num_q_heads=32,
                num_kv_heads=8, head_dim=128)
    c = DeviceCase(w)
    c.append()
    kb.kvpool_profile(True)
    out = c.forward(mirror=mirror)
    torch.cuda.synchronize()
    kb.kvpool_profile(False)
    assert "attn_reduce" not in kb.kernel_times(), "a call with no second split ran the reduce"
    assert_close(out_f64(out), c.oracle(), dtype, w.name, q_lens=w.q_lens)


# (context lengths, q_lens, q-heads, sparse parameters or None, pool dtype, reduce launches
# expected).  The reduce runs exactly when the shared split floor lets some sequence have a
# second split: 512 keys for single-tile rows (q_len * G <= 16, no sparse gap), otherwise 352 on
# bf16 pools and 256 on int8 pools; a sparse call may have a gap, so its host bound is 256.
REDUCE_CASES = [
    ([512, 300], [1, 1], 32, None, wl.BF16, 0),    # G = 4: 4 rows per KV head, 512-key splits
    ([513, 300], [1, 1], 32, None, wl.BF16, 1),    # 513 keys: a second split
    ([300, 200], [4, 1], 32, None, wl.BF16, 0),    # T*G = 16: still one tile, 512-key floor
    ([352, 200], [5, 1], 32, None, wl.BF16, 0),    # T*G = 20 on bf16: 352-key floor
    ([353, 200], [5, 1], 32, None, wl.BF16, 1),    # 353 keys: a second split
    ([300, 200], [5, 1], 32, None, wl.I8, 1),      # int8 pool: 256-key floor, 300 keys = 2 splits
    ([256, 100], [5, 2], 32, None, wl.I8, 0),      # 256-key floor but nobody past 256 keys
    ([400, 300], [1, 1], 32, (16, 64, 10**6), wl.BF16, 1),  # sparse, below threshold: bound 256
]


@pytest.mark.parametrize("case", range(len(REDUCE_CASES)))
def test_reduce_launch_follows_split_floor(case):
    """The host launches the reduce only when some sequence can have a second split, by the
    same floor the kernels split with; every row still matches the oracle."""
    ctx, ql, hq, sparse, dtype, expect = REDUCE_CASES[case]
    announce(f"reduce launch case {case}: ctx={ctx} q_lens={ql} sparse={sparse} {dtype}")
    w = wl.make(f"reduce_case_{case}", seed=170 + case, dtype=dtype, num_seqs_ctx=ctx,
                q_lens=ql, num_q_heads=hq, num_kv_heads=8, head_dim=128)
    c = DeviceCase(w)
    c.append()
    kb.kvpool_profile(True)
    out = c.forward(mirror=True) if sparse is None else c.forward_sparse(*sparse, mirror=True)
    torch.cuda.synchronize()
    kb.kvpool_profile(False)
    got = kb.kernel_times().get("attn_reduce", (0, 0.0))[0]
    assert got == expect, f"reduce launches {got}, expected {expect}"
    ref = c.oracle() if sparse is None else c.oracle_sparse(*sparse)
    assert_close(out_f64(out), ref, dtype, w.name, q_lens=w.q_lens)


@pytest.mark.parametrize("dtype,bs", [(wl.BF16, 16), (wl.BF16, 64), (wl.F32, 16)])
def test_nan_in_unread_slots(dtype, bs):
    """Pool starts all-NaN; the append writes exactly the context, so every slot past ctx_len and
    every unused block stays NaN; outputs must match the oracle run on the dense K/V."""
    announce(f"NaN canaries {dtype} B={bs}")
    ctx = [1, 15, 17, 100, 33]
    w = wl.make("nan", seed=71, dtype=dtype, num_seqs_ctx=ctx, q_lens=ctx, num_q_heads=8,
                num_kv_heads=2, head_dim=64, block_size=bs, num_blocks=sum((c + bs - 1) // bs for c in ctx) + 3)
    c = DeviceCase(w)
    c.pool.k_storage.fill_(float("nan"))
    c.pool.v_storage.fill_(float("nan"))
    c.append()
    torch.cuda.synchronize()
    # now attend with one query per sequence at the end of its context
    rng = np.random.default_rng(5)
    q = wl.draw(rng, (len(ctx), 8, 64), dtype)
    ql = torch.ones(len(ctx), dtype=torch.int32, device="cuda")
    out = c.pool.forward(0, to_torch(q, dtype), c.tables, c.ctx, ql, scale=w.scale)
    torch.cuda.synchronize()
    starts = np.concatenate([[0], np.cumsum(ctx)])
    ref = np.empty((len(ctx), 8, 64))
    for s, L in enumerate(ctx):
        kd = ora.to_f64(w.k_new[starts[s]:starts[s + 1]], dtype)
        vd = ora.to_f64(w.v_new[starts[s]:starts[s + 1]], dtype)
        ref[s] = ora.attention(ora.to_f64(q[s:s + 1], dtype), kd, vd, w.scale)[0]
    assert_close(out_f64(out), ref, dtype, "nan canaries")


def test_verify_rows_equal_decode_steps():
    announce("verify rows vs decode at their own lengths")
    L, T = 5000, 4
    w = wl.make("verify_vs_decode", seed=81, dtype=wl.BF16, num_seqs_ctx=[L], q_lens=[T],
                num_q_heads=40, num_kv_heads=8, head_dim=128)
    c = DeviceCase(w)
    c.append()
    ver = c.forward()
    for i in range(T):
        ctx = torch.tensor([L - T + i + 1], dtype=torch.int32, device="cuda")
        one = torch.ones(1, dtype=torch.int32, device="cuda")
        dec = c.pool.forward(0, c.q[i:i + 1], c.tables, ctx, one, scale=w.scale)
        torch.cuda.synchronize()
        assert_close(out_f64(dec), out_f64(ver[i:i + 1]), wl.BF16, f"row {i}")


def test_chunked_prefill_equals_one_pass():
    announce("suffix-only prefill over a cached prefix vs one pass")
    P, S = 1500, 548
    w = wl.make("oneshot", seed=91, dtype=wl.BF16, num_seqs_ctx=[P + S], q_lens=[P + S],
                num_q_heads=40, num_kv_heads=8, head_dim=128)
    c = DeviceCase(w)
    c.append()           # the whole prompt's K/V
    full = c.forward()   # one pass over every prompt row
    ql = torch.tensor([S], dtype=torch.int32, device="cuda")
    tail = c.pool.forward(0, c.q[P:], c.tables, c.ctx, ql, scale=w.scale)
    torch.cuda.synchronize()
    assert_close(out_f64(tail), out_f64(full[P:]), wl.BF16, "chunked vs one pass")


@pytest.mark.parametrize("split", ["32", "96", "4096", "16384"])
def test_forced_split_sizes(monkeypatch, split):
    """Fixed split sizes reach the 4-wave and block-id reload variants of the split kernel."""
    monkeypatch.setenv("KVATTN_SPLIT_TOKENS", split)
    announce(f"KVATTN_SPLIT_TOKENS={split}")
    w = wl.make(f"split{split}", seed=101, dtype=wl.BF16, num_seqs_ctx=[20000, 3001, 1, 70],
                q_lens=[1, 4, 1, 3], num_q_heads=40, num_kv_heads=8, head_dim=128)
    c = DeviceCase(w)
    c.append()
    out = c.forward()
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle(), wl.BF16, w.name, q_lens=w.q_lens)


@pytest.mark.parametrize("hq,hkv,d,bs", [(16, 1, 64, 64), (1, 1, 128, 16), (12, 4, 128, 64)])
def test_edge_shapes(hq, hkv, d, bs):
    announce(f"edge shapes Hq={hq} Hkv={hkv} D={d} B={bs}")
    w = wl.make("edge", seed=111, dtype=wl.BF16, num_seqs_ctx=[1, 5, 0, 64, 130, 7],
                q_lens=[1, 5, 0, 2, 0, 7], num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                block_size=bs)
    c = DeviceCase(w)
    c.append()
    out = c.forward()
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle(), wl.BF16, w.name, q_lens=w.q_lens)


def test_empty_batch_is_a_noop():
    announce("empty batch")
    pool = kb.PagedKVPool(1, 4, 16, 1, 64, kb.KV_BF16)
    z = torch.zeros(0, dtype=torch.int32, device="cuda")
    q = torch.zeros(0, 1, 64, dtype=torch.bfloat16, device="cuda")
    kb.kvattn_forward(pool.handle, 0, q, q, 1, 0.125, z, 1, z, z, 0, 0, 0, 0, None, 0)
    kb.kvpool_append(pool.handle, 0, q, q, z, 1, z, z, 0, 0, 0)
    kb.kvpool_copy_blocks(pool.handle, z, z, 0)


# ---------------------------------------------------------------------------------------------
# Host-side validation (KVPOOL_VALIDATE=1): every violation is refused with its code
# ---------------------------------------------------------------------------------------------

def _small():
    w = wl.make("val", seed=121, dtype=wl.BF16, num_seqs_ctx=[40, 17], q_lens=[2, 1],
                num_q_heads=4, num_kv_heads=2, head_dim=64, num_blocks=8)
    return w, DeviceCase(w)


def _expect(code, fn):
    with pytest.raises(kb.KVPoolError) as e:
        fn()
    assert e.value.code == code, (e.value.code, str(e.value))


def test_validation_codes(monkeypatch):
    announce("validation error codes")
    monkeypatch.setenv("KVPOOL_VALIDATE", "1")
    w, c = _small()
    c.append()
    c.forward()  # valid metadata passes validation
    bad = c.tables.clone()
    bad[0, 0] = 99
    _expect(kb.KV_ERANGE, lambda: c.pool.forward(0, c.q, bad, c.ctx, c.ql, scale=w.scale))
    _expect(kb.KV_ERANGE, lambda: c.pool.append(0, c.k_new, c.v_new, bad, c.ctx, c.ql))
    neg = c.tables.clone()
    neg[1, 1] = -1
    _expect(kb.KV_ERANGE, lambda: c.pool.forward(0, c.q, neg, c.ctx, c.ql, scale=w.scale))
    ql_big = torch.tensor([41, 1], dtype=torch.int32, device="cuda")
    _expect(kb.KV_ERANGE, lambda: c.pool.forward(0, torch.empty(42, 4, 64, dtype=torch.bfloat16, device="cuda"),
                                                 c.tables, c.ctx, ql_big, scale=w.scale,
                                                 max_ctx_len=48, max_q_len=41))
    ctx_big = torch.tensor([40, 17 + 16 * 5], dtype=torch.int32, device="cuda")
    _expect(kb.KV_ERANGE, lambda: c.pool.forward(0, c.q, c.tables, ctx_big, c.ql, scale=w.scale))
    # max_ctx_len below a sequence's length
    _expect(kb.KV_ERANGE, lambda: c.pool.forward(0, c.q, c.tables, c.ctx, c.ql, scale=w.scale,
                                                 max_ctx_len=20))
    # sum(q_lens) != total_q
    _expect(kb.KV_ERANGE, lambda: c.pool.forward(0, c.q[:2], c.tables, c.ctx, c.ql, scale=w.scale))
    # a host mirror of q_lens that differs from the device q_lens
    _expect(kb.KV_ERANGE, lambda: c.pool.forward(0, c.q, c.tables, c.ctx, c.ql, scale=w.scale,
                                                 q_lens_host=[1, 2]))
    c.pool.forward(0, c.q, c.tables, c.ctx, c.ql, scale=w.scale, q_lens_host=w.q_lens)
    # two sequences writing the same block
    shared = c.tables.clone()
    shared[1, 1] = shared[0, 2]
    _expect(kb.KV_ERANGE, lambda: c.pool.append(0, c.k_new, c.v_new, shared, c.ctx, c.ql))
    # copy_blocks: repeated dst, dst also a src, id out of range
    t = lambda *v: torch.tensor(v, dtype=torch.int32, device="cuda")  # noqa: E731
    _expect(kb.KV_ERANGE, lambda: c.pool.copy_blocks(t(0, 1), t(5, 5)))
    _expect(kb.KV_ERANGE, lambda: c.pool.copy_blocks(t(0, 1), t(1, 6)))
    _expect(kb.KV_ERANGE, lambda: c.pool.copy_blocks(t(0), t(8)))


def test_argument_codes():
    announce("argument error codes")
    w, c = _small()
    h = c.pool.handle
    ws, need = c.pool.workspace(4, 2, 3, 40, 2)
    args = lambda **o: dict(dict(handle=h, layer=0, q=c.q, out=c.q.clone(), num_q_heads=4, scale=w.scale,  # noqa: E731
                                 block_tables=c.tables, max_blocks_per_seq=c.tables.shape[1],
                                 ctx_lens=c.ctx, q_lens=c.ql, num_seqs=2, total_q=3,
                                 max_ctx_len=40, max_q_len=2, workspace=ws, workspace_bytes=need), **o)
    kb.kvattn_forward(**args())
    _expect(kb.KV_EINVAL, lambda: kb.kvattn_forward(**args(layer=1)))
    _expect(kb.KV_EINVAL, lambda: kb.kvattn_forward(**args(num_q_heads=5)))
    _expect(kb.KV_EUNSUPPORTED, lambda: kb.kvattn_forward(**args(num_q_heads=34)))
    _expect(kb.KV_EINVAL, lambda: kb.kvattn_forward(**args(scale=float("inf"))))
    _expect(kb.KV_EINVAL, lambda: kb.kvattn_forward(**args(q=c.q.view(-1)[1:].data_ptr())))
    if need:
        _expect(kb.KV_ENOMEM, lambda: kb.kvattn_forward(**args(workspace_bytes=need - 1)))
        _expect(kb.KV_ENOMEM, lambda: kb.kvattn_forward(**args(workspace=None)))
    _expect(kb.KV_EINVAL, lambda: kb.kvattn_forward(**args(max_q_len=41)))
    with pytest.raises(kb.KVPoolError) as e:
        kb.PagedKVPool(1, 4, 32, 1, 64, kb.KV_BF16)
    assert e.value.code == kb.KV_EUNSUPPORTED


@pytest.mark.parametrize("mode", ["decode_verify", "prefill"])
def test_graph_replay_matches_eager(mode):
    """append + attention captured in a HIP graph: every replay, with other GPU work between
    replays, equals the eager result bit for bit (the library records no memset and makes no
    host synchronisation)."""
    announce(f"HIP graph replay {mode}")
    if mode == "decode_verify":
        w = wl.make("graph", **MIXED)
    else:
        w = wl.make("graph_pf", seed=131, dtype=wl.BF16, num_seqs_ctx=[700, 300], q_lens=[300, 100],
                    num_q_heads=40, num_kv_heads=8, head_dim=128)
    c = DeviceCase(w)
    c.append()
    eager = c.forward().clone()
    out = torch.empty_like(c.q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        c.forward(out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        c.append()
        c.forward(out=out)
    junk = torch.randn(1 << 20, device="cuda")
    for i in range(4):
        out.fill_(float("nan"))
        junk.mul_(1.0001).sum()           # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), bits(eager)), f"replay {i}"


@pytest.mark.parametrize("dtype", [wl.BF16, wl.F32])
def test_default_mode_decode_rows_batch_invariant(dtype, monkeypatch):
    """Without deterministic mode the prefill plan follows the batch, but decode and verification
    rows (the split-K path: no plan choice) still give each sequence's bits alone; every row
    stays within tolerance of the oracle."""
    monkeypatch.delenv("KVATTN_DETERMINISTIC", raising=False)
    announce(f"default-mode invariance of split-K rows {dtype}")
    w = wl.make("mixed_inv_default", seed=152, dtype=dtype,
                num_seqs_ctx=[3000, 700, 1000, 9000, 129, 40, 5000],
                q_lens=[1, 4, 300, 4, 129, 33, 1], num_q_heads=40, num_kv_heads=8, head_dim=128)
    c = DeviceCase(w)
    c.append()
    full = c.forward()
    torch.cuda.synchronize()
    assert_close(out_f64(full), c.oracle(), dtype, w.name, q_lens=w.q_lens)
    starts = np.concatenate([[0], np.cumsum(w.q_lens)])
    G = w.num_q_heads // w.num_kv_heads
    for s in range(w.num_seqs):
        if w.q_lens[s] * G > 128:
            continue  # a prefill-class sequence: its plan follows the batch in this mode
        rows = slice(int(starts[s]), int(starts[s + 1]))
        sel = torch.tensor([s], device="cuda")
        alone = c.pool.forward(0, c.q[rows], c.tables[sel], c.ctx[sel], c.ql[sel], scale=w.scale,
                               max_ctx_len=int(w.ctx_lens[s]), max_q_len=int(w.q_lens[s]))
        torch.cuda.synchronize()
        assert np.array_equal(bits(alone), bits(full[rows])), f"sequence {s}"
