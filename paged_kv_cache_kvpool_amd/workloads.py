"""Seeded synthetic inputs for paged-KV attention (shared by the oracle side and the HIP side).

This module only draws numbers. It holds none of the attention arithmetic and none of the
pool's intra-block layout: pools are produced as raw storage (one flat row of
``num_kv_heads * block_size * head_dim`` elements per block), so whatever reads a pool must
apply the layout itself.

Shapes follow the pages' serving setting: a block-paged KV pool shared by all sequences and
sized once (sparkinfer server README, "Serve Qwen3.8 with DSpark"; NInfer serving doc,
"Execution behavior"), 16-token blocks (sparkinfer README, "Automatic prefix cache"),
GQA heads, decode batches, speculative verification of 1 + k draft tokens and prefix-reuse
prefill where only the uncached suffix is new.

Recipe (the same for every generator):
  * values ~ N(0, 1) drawn as float32 by ``numpy.random.default_rng(seed)`` (PCG64);
    bf16 values are the round-to-nearest-even bf16 of those float32 draws, kept as uint16 bits;
  * pool blocks that no block table references hold NaN canaries (whole blocks);
  * block tables are slices of one seeded permutation of the pool, so placement is random
    and sequences never share a block unless a test asks for it;
  * the K/V of tokens being processed (``k_new``/``v_new``) are drawn separately and are
    written by the append call before attention;
  * int8 pools are drawn as raw storage too: codes round(N(0,1) * 127 / 4) clipped to +-127 and
    scales 4/127 * U(0.8, 1.2) (dequantized values roughly N(0, 1)); unreferenced blocks carry
    NaN scales as canaries.  q and the new rows of an int8 pool are bf16.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"
I8 = "i8"     # int8 pool: codes and per-(token, KV head) fp32 scales; q and new rows are bf16

BF16_NAN = np.uint16(0x7FC0)
F32_NAN = np.float32(np.nan)


def rne_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def draw(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) values in the storage dtype (float32 array, or uint16 bf16 bits)."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return x if dtype == F32 else rne_bf16_bits(x)


def nan_fill(dtype: str):
    return F32_NAN if dtype == F32 else BF16_NAN


@dataclasses.dataclass
class Workload:
    """One call's worth of inputs.  Arrays are numpy; bf16 arrays hold uint16 bits."""

    name: str
    dtype: str
    num_layers: int
    num_blocks: int
    block_size: int
    num_kv_heads: int
    num_q_heads: int
    head_dim: int
    scale: float
    layer: int
    q: np.ndarray                 # [total_q, Hq, D]
    k_pool: Optional[np.ndarray]  # [num_layers, num_blocks, Hkv*B*D] raw storage (None: see pool_seed)
    v_pool: Optional[np.ndarray]
    block_tables: np.ndarray      # int32 [S, max_blocks]
    ctx_lens: np.ndarray          # int32 [S]  (counts the tokens being processed)
    q_lens: np.ndarray            # int32 [S]
    k_new: Optional[np.ndarray] = None   # [total_q, Hkv, D]: appended before attention
    v_new: Optional[np.ndarray] = None
    pool_seed: Optional[int] = None      # set when the pool is too large to draw on the host
    referenced: Optional[np.ndarray] = None  # bool [num_blocks]: blocks some table uses
    k_scales: Optional[np.ndarray] = None    # int8 pools: float32 [layers][blocks][Hkv][B]
    v_scales: Optional[np.ndarray] = None
    sparse: Optional[tuple] = None  # (sink, window, min_len): run as sink + window sparse attention

    @property
    def num_seqs(self) -> int:
        return int(self.ctx_lens.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.q_lens.sum())

    @property
    def block_elems(self) -> int:
        return self.num_kv_heads * self.block_size * self.head_dim

    @property
    def elt_bytes(self) -> int:
        """Bytes of one pool element."""
        return 4 if self.dtype == F32 else 1 if self.dtype == I8 else 2

    @property
    def act_dtype(self) -> str:
        """dtype of q, out and the new rows (bf16 for an int8 pool)."""
        return BF16 if self.dtype == I8 else self.dtype


def _blocks_for(ctx: int, block_size: int) -> int:
    return (int(ctx) + block_size - 1) // block_size


def _tables_from_perm(perm: np.ndarray, ctx_lens, block_size: int, max_blocks: Optional[int] = None):
    """Cut one permutation of pool block ids into consecutive per-sequence slices."""
    need = [_blocks_for(c, block_size) for c in ctx_lens]
    width = max(need) if max_blocks is None else max_blocks
    tables = np.zeros((len(ctx_lens), width), dtype=np.int32)
    pos = 0
    for s, n in enumerate(need):
        tables[s, :n] = perm[pos:pos + n]
        pos += n
    return tables, pos


def _pool(rng, dtype, num_layers, num_blocks, block_elems, referenced):
    k = draw(rng, (num_layers, num_blocks, block_elems), dtype)
    v = draw(rng, (num_layers, num_blocks, block_elems), dtype)
    k[:, ~referenced] = nan_fill(dtype)
    v[:, ~referenced] = nan_fill(dtype)
    return k, v


def draw_codes(rng, shape) -> np.ndarray:
    """int8 codes round(N(0,1) * 127 / 4), clipped to +-127."""
    x = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(127.0 / 4.0)
    return np.clip(np.rint(x), -127, 127).astype(np.int8)


def draw_scales(rng, shape) -> np.ndarray:
    return (rng.uniform(0.8, 1.2, size=shape) * (4.0 / 127.0)).astype(np.float32)


def _pool_i8(rng, num_layers, num_blocks, num_kv_heads, block_size, head_dim, referenced):
    elems = num_kv_heads * block_size * head_dim
    k = draw_codes(rng, (num_layers, num_blocks, elems))
    v = draw_codes(rng, (num_layers, num_blocks, elems))
    sshape = (num_layers, num_blocks, num_kv_heads, block_size)
    ks, vs = draw_scales(rng, sshape), draw_scales(rng, sshape)
    ks[:, ~referenced] = np.nan
    vs[:, ~referenced] = np.nan
    return k, v, ks, vs


def _referenced(tables, ctx_lens, block_size, num_blocks):
    ref = np.zeros(num_blocks, dtype=bool)
    for s, c in enumerate(ctx_lens):
        ref[tables[s, :_blocks_for(c, block_size)]] = True
    return ref


def make(name, *, seed, dtype, num_seqs_ctx, q_lens, num_q_heads, num_kv_heads, head_dim,
         block_size=16, num_blocks=None, num_layers=1, layer=0, scale=None, append=True,
         host_pool=True, max_blocks=None) -> Workload:
    """General generator.

    ``num_seqs_ctx``: ctx_len per sequence (already counting the q_len new tokens).
    ``append``: draw k_new/v_new for the q_len new tokens of each sequence (written by the
    append call before attention); otherwise the pool already holds them.
    ``host_pool=False`` leaves the pool undrawn (``pool_seed`` set) so a device-side
    generator can fill it; used for pools of hundreds of MB.
    """
    rng = np.random.default_rng(seed)
    ctx = np.asarray(num_seqs_ctx, dtype=np.int32)
    ql = np.asarray(q_lens, dtype=np.int32)
    assert ctx.shape == ql.shape and np.all(ql <= ctx) and np.all(ql >= 0)
    need = int(sum(_blocks_for(c, block_size) for c in ctx))
    nb = need if num_blocks is None else int(num_blocks)
    assert nb >= need
    perm = rng.permutation(nb).astype(np.int32)
    tables, _ = _tables_from_perm(perm, ctx, block_size, max_blocks)
    total_q = int(ql.sum())
    act = BF16 if dtype == I8 else dtype
    q = draw(rng, (total_q, num_q_heads, head_dim), act)
    k_new = v_new = None
    if append:
        k_new = draw(rng, (total_q, num_kv_heads, head_dim), act)
        v_new = draw(rng, (total_q, num_kv_heads, head_dim), act)
    ref = _referenced(tables, ctx, block_size, nb)
    block_elems = num_kv_heads * block_size * head_dim
    k_pool = v_pool = k_scales = v_scales = None
    pool_seed = None
    if host_pool and dtype == I8:
        k_pool, v_pool, k_scales, v_scales = _pool_i8(rng, num_layers, nb, num_kv_heads,
                                                      block_size, head_dim, ref)
    elif host_pool:
        k_pool, v_pool = _pool(rng, dtype, num_layers, nb, block_elems, ref)
    else:
        pool_seed = int(rng.integers(0, 2**31 - 1))
    if scale is None:
        scale = 1.0 / float(np.sqrt(head_dim))
    return Workload(name=name, dtype=dtype, num_layers=num_layers, num_blocks=nb,
                    block_size=block_size, num_kv_heads=num_kv_heads, num_q_heads=num_q_heads,
                    head_dim=head_dim, scale=float(scale), layer=layer, q=q, k_pool=k_pool,
                    v_pool=v_pool, block_tables=tables, ctx_lens=ctx, q_lens=ql, k_new=k_new,
                    v_new=v_new, pool_seed=pool_seed, referenced=ref, k_scales=k_scales,
                    v_scales=v_scales)


# ---------------------------------------------------------------------------------------
# The five workloads the method is measured on
# ---------------------------------------------------------------------------------------

def tiny_decode(seed: int = 0) -> Workload:
    """1 sequence, 1 query token, 1/1 heads, D=64, fp32, context 256 = 16 blocks of 16 placed
    by a random permutation of a 32-block pool (the other 16 blocks are NaN), scale 1/8."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(32).astype(np.int32)
    tables = perm[:16].reshape(1, 16).copy()
    ref = np.zeros(32, dtype=bool)
    ref[tables[0]] = True
    q = draw(rng, (1, 1, 64), F32)
    k, v = _pool(rng, F32, 1, 32, 1 * 16 * 64, ref)
    return Workload(name="tiny_decode", dtype=F32, num_layers=1, num_blocks=32, block_size=16,
                    num_kv_heads=1, num_q_heads=1, head_dim=64, scale=1.0 / 8.0, layer=0, q=q,
                    k_pool=k, v_pool=v, block_tables=tables,
                    ctx_lens=np.array([256], np.int32), q_lens=np.array([1], np.int32),
                    referenced=ref)


def batched_gqa_decode(seed: int = 1, num_seqs: int = 32, host_pool: bool = True,
                       dtype: str = BF16) -> Workload:
    """32 sequences x 1 query token, 32 q-heads / 8 kv-heads, D=128, bf16, B=16, contexts
    uniform on [1024, 8192]; the pool is exactly the blocks the contexts need, dealt out as
    disjoint random slices of one permutation.  The current token's K/V is appended first."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(1024, 8193, size=num_seqs).astype(np.int32)
    return make("batched_gqa_decode" + ("_int8" if dtype == I8 else ""), seed=seed + 1000,
                dtype=dtype, num_seqs_ctx=ctx, q_lens=np.ones(num_seqs, np.int32),
                num_q_heads=32, num_kv_heads=8, head_dim=128, append=True, host_pool=host_pool)


def spec_verify(seed: int = 2, cached: int = 32768, drafts: int = 3,
                host_pool: bool = True, dtype: str = BF16) -> Workload:
    """One sequence verifying 1 + drafts tokens (causal among themselves) over a cached
    context, 40 q-heads / 8 kv-heads, D=128, bf16, randomly permuted table; the new tokens'
    K/V are appended at positions cached .. cached+drafts."""
    t = 1 + drafts
    return make(f"spec_verify_{cached}" + ("_int8" if dtype == I8 else ""), seed=seed,
                dtype=dtype, num_seqs_ctx=[cached + t],
                q_lens=[t], num_q_heads=40, num_kv_heads=8, head_dim=128, append=True,
                host_pool=host_pool)


def prefix_prefill(seed: int = 3, num_seqs: int = 4, prefix: int = 4096, suffix: int = 512,
                   host_pool: bool = True, dtype: str = BF16) -> Workload:
    """4 sequences, each a 4096-token cached prefix plus a 512-token new suffix (causal),
    40/8 heads, D=128, bf16; the suffix K/V are appended before attention."""
    return make("prefix_prefill" + ("_int8" if dtype == I8 else ""), seed=seed, dtype=dtype,
                num_seqs_ctx=[prefix + suffix] * num_seqs, q_lens=[suffix] * num_seqs,
                num_q_heads=40, num_kv_heads=8, head_dim=128, append=True, host_pool=host_pool)


def long_prefix_chunk(seed: int = 7, prefix: int = 32768, suffix: int = 512,
                      host_pool: bool = True, dtype: str = BF16) -> Workload:
    """One chunked-prefill step of a long prompt: a 512-token chunk over a 32768-token cached
    prefix (causal), 40/8 heads, D=128, bf16.  Its row tiles alone fill under two thirds of the
    GPU, so each row tile's keys are cut into ranges."""
    return make("long_prefix_chunk" + ("_int8" if dtype == I8 else ""), seed=seed, dtype=dtype,
                num_seqs_ctx=[prefix + suffix], q_lens=[suffix], num_q_heads=40, num_kv_heads=8,
                head_dim=128, append=True, host_pool=host_pool)


def long_decode(seed: int = 4, host_pool: bool = False, dtype: str = BF16) -> Workload:
    """2 concurrent sequences at 262144 and 131072 tokens, 1 query token each, 40/8 heads,
    D=128, bf16, pool of 24576 blocks (393216 tokens) with random placement."""
    return make("long_decode" + ("_int8" if dtype == I8 else ""), seed=seed, dtype=dtype,
                num_seqs_ctx=[262144, 131072],
                q_lens=[1, 1], num_q_heads=40, num_kv_heads=8, head_dim=128, append=True,
                num_blocks=24576, host_pool=host_pool)


def mixed_step(seed: int = 5, host_pool: bool = True, dtype: str = BF16) -> Workload:
    """One serving step that batches every kind of sequence the pool serves: 32 decode
    sequences (1 token, contexts uniform on [1024, 8192]), one verification of 1 + 3 draft
    tokens over a 32768-token context and one 512-token prefill chunk over a 4096-token cached
    prefix; 40/8 heads, D=128, bf16, B=16.  New tokens' K/V are appended first."""
    rng = np.random.default_rng(seed)
    ctx = list(rng.integers(1024, 8193, size=32).astype(np.int32))
    ql = [1] * 32
    # the verification and the prefill chunk sit between decode sequences
    ctx[10:10] = [32768 + 4]
    ql[10:10] = [4]
    ctx[20:20] = [4096 + 512]
    ql[20:20] = [512]
    return make("mixed_step" + ("_int8" if dtype == I8 else ""), seed=seed + 1000, dtype=dtype,
                num_seqs_ctx=ctx, q_lens=ql,
                num_q_heads=40, num_kv_heads=8, head_dim=128, append=True, host_pool=host_pool)


# The pages' sparse decode mode: the first KV block (16 tokens) and the last 4096 tokens once a
# sequence holds 16384 (sparkinfer server README, "Env", SPARKINFER_SPARSE_GQA6).
PAGES_SPARSE = (16, 4096, 16384)


def sparse_decode(seed: int = 6, num_seqs: int = 32, host_pool: bool = False,
                  dtype: str = BF16) -> Workload:
    """32 sequences x 1 query token with contexts uniform on [16384, 65536], 32/8 heads, D=128,
    bf16, B=16, in the pages' sparse mode (each reads 16 + 4096 keys); the pool holds every
    context in full (drawn on the device)."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(16384, 65537, size=num_seqs).astype(np.int32)
    w = make("sparse_decode" + ("_int8" if dtype == I8 else ""), seed=seed + 1000, dtype=dtype,
             num_seqs_ctx=ctx, q_lens=np.ones(num_seqs, np.int32), num_q_heads=32,
             num_kv_heads=8, head_dim=128, append=True, host_pool=host_pool)
    w.sparse = PAGES_SPARSE
    return w


def long_decode_sparse(seed: int = 4, dtype: str = BF16) -> Workload:
    """The long-context decode workload (262144 and 131072 keys) in the pages' sparse mode."""
    w = long_decode(seed=seed, dtype=dtype)
    w.name = "long_decode_sparse" + ("_int8" if dtype == I8 else "")
    w.sparse = PAGES_SPARSE
    return w


def random_case(seed: int, *, dtype=BF16, num_seqs=3, num_q_heads=8, num_kv_heads=2,
                head_dim=64, block_size=16, q_len_choices=(1, 2, 4, 17), max_ctx=300,
                extra_blocks=5, append=True) -> Workload:
    """Small seeded case for parity sweeps: ragged contexts (including shorter than one block
    and not a multiple of the block size), mixed query lengths, spare NaN blocks."""
    rng = np.random.default_rng(seed + 7919)
    ql = rng.choice(np.asarray(q_len_choices), size=num_seqs).astype(np.int32)
    ctx = np.array([int(rng.integers(int(t), max(int(t), max_ctx) + 1)) for t in ql], np.int32)
    need = sum(_blocks_for(c, block_size) for c in ctx)
    return make(f"random_{seed}", seed=seed, dtype=dtype, num_seqs_ctx=ctx, q_lens=ql,
                num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                block_size=block_size, num_blocks=need + extra_blocks, append=append)
