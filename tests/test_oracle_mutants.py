"""Plant plausible mistakes in the oracle (CPU only) and require that some pin catches each.

This shows the pins are strong enough: a dropped term, a wrong index, sign or axis, or a
misread storage layout in the oracle fails at least one of them.
"""
import numpy as np
import pytest

from oracle import attention as ora
from tests import oracle_pins as pins

_real_attention = ora.attention
_real_gather = ora.gather_kv
_real_append = ora.append
_real_copy = ora.copy_blocks


def _attn_variant(*, shift=0, top_left=False, head_mod=False, scale_mul=1.0, use_k_for_v=False,
                  sum_axis=1, include_diag=True, no_scale=False):
    def attention(q, k, v, scale):
        t_len, hq, _ = q.shape
        l_len, hkv, _ = k.shape
        group = hq // hkv
        out = np.empty(q.shape)
        base = 0 if top_left else (l_len - t_len)
        pos = base + np.arange(t_len)[:, None] + shift
        j = np.arange(l_len)[None, :]
        masked = (j > pos) if include_diag else (j >= pos)
        for h in range(hq):
            g = (h % hkv) if head_mod else (h // group)
            eff = 1.0 if no_scale else scale * scale_mul
            s = eff * (q[:, h, :] @ k[:, g, :].T)
            s = np.where(masked, -np.inf, s)
            w = np.exp(s - s.max(axis=1, keepdims=True))
            vv = k[:, g, :] if use_k_for_v else v[:, g, :]
            den = w.sum(axis=sum_axis, keepdims=True)
            if sum_axis == 0:
                den = den.sum()
            out[:, h, :] = (w @ vv) / den
        return out
    return attention


def _gather_k_untransposed(k_pool, v_pool, layer, table_row, ctx_len, *, num_kv_heads,
                           block_size, head_dim, dtype):
    """Reads K as if it were stored [t][d] (ignores the 16-byte chunk tiling)."""
    k, v = _real_gather(k_pool, v_pool, layer, table_row, ctx_len, num_kv_heads=num_kv_heads,
                        block_size=block_size, head_dim=head_dim, dtype=dtype)
    nblk = (int(ctx_len) + block_size - 1) // block_size
    ks = [k_pool[layer, int(table_row[j])].reshape(num_kv_heads, block_size, head_dim)
          .transpose(1, 0, 2) for j in range(nblk)]
    return np.concatenate(ks)[:ctx_len], v


def _gather_v_untransposed(k_pool, v_pool, layer, table_row, ctx_len, *, num_kv_heads,
                           block_size, head_dim, dtype):
    """Reads V as if it were stored [t][d] instead of dims-major."""
    k, _ = _real_gather(k_pool, v_pool, layer, table_row, ctx_len, num_kv_heads=num_kv_heads,
                        block_size=block_size, head_dim=head_dim, dtype=dtype)
    nblk = (int(ctx_len) + block_size - 1) // block_size
    vs = [v_pool[layer, int(table_row[j])].reshape(num_kv_heads, block_size, head_dim)
          .transpose(1, 0, 2) for j in range(nblk)]
    return k, np.concatenate(vs)[:ctx_len]


def _gather_no_trim(k_pool, v_pool, layer, table_row, ctx_len, **kw):
    """Forgets to cut the last block at ctx_len (reads the tail slots)."""
    bs = kw["block_size"]
    full = (int(ctx_len) + bs - 1) // bs * bs
    return _real_gather(k_pool, v_pool, layer, list(table_row) + [0], full, **kw)


def _gather_wrong_block(k_pool, v_pool, layer, table_row, ctx_len, **kw):
    """Uses the physical id of block j for every block after the first (stale table read)."""
    row = list(table_row)
    row = [row[0]] * len(row)
    return _real_gather(k_pool, v_pool, layer, row, ctx_len, **kw)


def _append_off_by_one(k_pool, v_pool, layer, k_new, v_new, tables, ctx_lens, q_lens, **kw):
    return _real_append(k_pool, v_pool, layer, k_new, v_new, tables, ctx_lens + 1, q_lens, **kw)


def _copy_swapped(k_pool, v_pool, src, dst):
    return _real_copy(k_pool, v_pool, dst, src)


MUTANTS = [
    ("mask_shift_plus1", "attention", _attn_variant(shift=1)),
    ("mask_excludes_diagonal", "attention", _attn_variant(include_diag=False)),
    ("top_left_alignment", "attention", _attn_variant(top_left=True)),
    ("gqa_head_modulo", "attention", _attn_variant(head_mod=True)),
    ("no_scale", "attention", _attn_variant(no_scale=True)),
    ("double_scale", "attention", _attn_variant(scale_mul=2.0)),
    ("k_used_as_v", "attention", _attn_variant(use_k_for_v=True)),
    ("normalise_wrong_axis", "attention", _attn_variant(sum_axis=0)),
    ("gather_k_untiled", "gather_kv", _gather_k_untransposed),
    ("gather_v_untransposed", "gather_kv", _gather_v_untransposed),
    ("gather_reads_tail", "gather_kv", _gather_no_trim),
    ("gather_wrong_block", "gather_kv", _gather_wrong_block),
    ("append_off_by_one", "append", _append_off_by_one),
    ("copy_src_dst_swapped", "copy_blocks", _copy_swapped),
]


@pytest.mark.parametrize("name,attr,fn", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(monkeypatch, name, attr, fn):
    monkeypatch.setattr(ora, attr, fn)
    caught = []
    for pin_name, pin, kw in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(**kw)
        except (AssertionError, IndexError, ValueError, FloatingPointError):
            caught.append(pin_name)
    assert caught, f"no pin catches the planted mistake {name}"
