"""Sink + window sparse attention, written out plainly.

TEST INFRASTRUCTURE: see the package docstring.

The pages offer a decode mode that, once a sequence holds 16384 tokens, attends only to the
sequence's first KV block and its most recent 4096 tokens, and to nothing in between
(sparkinfer server README, "Env", SPARKINFER_SPARSE_GQA6).  Readings taken:

* the rule is applied per query row: a row at absolute position p sees p + 1 keys when dense;
  if p + 1 >= min_len it sees only the keys j <= p with j < sink or j >= p + 1 - window, i.e.
  the first `sink` positions and the `window` most recent ones including its own.  For a
  decode row (p = L - 1) this is exactly the pages' rule with sink = one block, window = 4096,
  min_len = 16384; verification rows get the same rule each, at their own positions;
* "the first KV block" is the sequence's first block_size positions (sink = block_size); the
  three numbers are parameters with the pages' values as the usual choice;
* a row with p + 1 < min_len is dense; where the sink and the window overlap they are simply
  united.

Everything else (scale, GQA mapping, bottom-right alignment, the pool layouts) is that of
``oracle.attention`` and ``oracle.quant``.
"""
from __future__ import annotations

import numpy as np

from . import attention as ora
from . import quant as oq


def visible(p: int, l_len: int, *, sink: int, window: int, min_len: int) -> np.ndarray:
    """Boolean mask over keys 0 .. l_len - 1 of what a row at absolute position p sees."""
    j = np.arange(l_len)
    seen = j <= p
    if p + 1 >= min_len:
        seen &= (j < sink) | (j >= p + 1 - window)
    return seen


def attention(q, k, v, scale, *, sink, window, min_len):
    """As ``oracle.attention.attention`` (T query rows at the last T of L positions), with each
    row restricted to the keys ``visible`` gives it.  q [T, Hq, D], k, v [L, Hkv, D] float64."""
    t_len, hq, _ = q.shape
    l_len, hkv, _ = k.shape
    assert hq % hkv == 0 and 1 <= t_len <= l_len and window >= 1 and sink >= 0
    group = hq // hkv
    seen = np.stack([visible(l_len - t_len + i, l_len, sink=sink, window=window,
                             min_len=min_len) for i in range(t_len)])  # [T, L]
    out = np.empty(q.shape, dtype=np.float64)
    for h in range(hq):
        g = h // group
        s = scale * (q[:, h, :] @ k[:, g, :].T)
        s = np.where(seen, s, -np.inf)
        w = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h, :] = (w @ v[:, g, :]) / w.sum(axis=1, keepdims=True)
    return out


def paged_attention(q, k_pool, v_pool, layer, block_tables, ctx_lens, q_lens, *, scale,
                    num_kv_heads, block_size, head_dim, dtype, sink, window, min_len,
                    scales=None, seqs=None):
    """Sparse attention for a packed batch.  dtype "f32" / "bf16" pools as in
    ``oracle.attention``; dtype "i8" pools as in ``oracle.quant`` with ``scales`` = (K scales,
    V scales) and bf16 q.  Returns float64 [sum(q_lens), Hq, D]."""
    i8 = dtype == "i8"
    qf = ora.to_f64(q, "bf16" if i8 else dtype)
    out = np.full(qf.shape, np.nan)
    starts = np.concatenate([[0], np.cumsum(np.asarray(q_lens, dtype=np.int64))])
    geo = dict(num_kv_heads=num_kv_heads, block_size=block_size, head_dim=head_dim)
    todo = range(len(ctx_lens)) if seqs is None else seqs
    for s in todo:
        t_len, l_len = int(q_lens[s]), int(ctx_lens[s])
        if t_len == 0:
            continue
        if i8:
            k, v = oq.gather_kv(k_pool, v_pool, scales[0], scales[1], layer, block_tables[s],
                                l_len, **geo)
        else:
            kb, vb = ora.gather_kv(k_pool, v_pool, layer, block_tables[s], l_len, dtype=dtype,
                                   **geo)
            k, v = ora.to_f64(kb, dtype), ora.to_f64(vb, dtype)
        rows = slice(int(starts[s]), int(starts[s]) + t_len)
        out[rows] = attention(qf[rows], k, v, scale, sink=sink, window=window, min_len=min_len)
    return out
