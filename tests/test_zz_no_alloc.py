"""kvattn_forward_noalloc (the entry point for callers that cannot allocate: its workspace is the
library's static per-GPU scratch) against kvattn_forward with a caller workspace, through the C
ABI: two calls in a row, the second smaller, each bit for bit the workspace call's output and
within the oracle's tolerance; a call needing more scratch than the buffer holds is refused."""
import sys

import numpy as np
import pytest
import torch

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


# (name, contexts, q_lens): a mixed call (decode, verification, a prefill chunk) first, then a
# smaller decode + verification call on the same GPU's scratch.
CALLS = [
    ("noalloc_mixed", [5000, 1200, 3000, 4700, 700, 2600], [1, 4, 1, 40, 1, 4]),
    ("noalloc_small", [900, 2100], [1, 4]),
]


def run_pair(name, ctx, ql, mirror):
    w = wl.make(name, seed=211 + len(ctx), dtype=wl.BF16, num_seqs_ctx=ctx, q_lens=ql,
                num_q_heads=32, num_kv_heads=8, head_dim=128)
    c = DeviceCase(w)
    c.append()
    torch.cuda.synchronize()
    ref_ws = c.forward(mirror=mirror)  # kvattn_forward, caller workspace
    out = torch.empty_like(c.q)
    out.fill_(float("nan"))
    torch.cuda.synchronize()
    c.pool.forward_noalloc(w.layer, c.q, c.tables, c.ctx, c.ql, int(w.ctx_lens.max()),
                           int(w.q_lens.max()), out, scale=w.scale,
                           q_lens_host=w.q_lens if mirror else None)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), bits(ref_ws)), f"{name}: bits differ from kvattn_forward"
    assert_close(out_f64(out), c.oracle(), wl.BF16, name, q_lens=w.q_lens)


@pytest.mark.parametrize("mirror", [True, False], ids=["mirror", "bounds"])
def test_noalloc_matches_workspace_call(mirror):
    for name, ctx, ql in CALLS:  # two calls in a row, the second smaller
        announce(f"{name} mirror={mirror}")
        run_pair(name, ctx, ql, mirror)


def test_noalloc_int8_prefill_without_room_for_the_copy():
    """An int8 prefill whose bf16 copy (about 147 MB here) exceeds the static buffer still runs
    on the allocation-free entry point: the prefill kernel converts the codes in LDS, with the
    same bits as kvattn_forward with a workspace that holds the copy; sampled rows against the
    oracle."""
    announce("noalloc int8 prefill, copy larger than the static buffer")
    w = wl.make("noalloc_i8_long", seed=233, dtype=wl.I8, num_seqs_ctx=[36000], q_lens=[64],
                num_q_heads=40, num_kv_heads=8, head_dim=128)
    c = DeviceCase(w)
    c.append()
    torch.cuda.synchronize()
    need = kb.kvattn_workspace_size(c.pool.handle, 40, 1, 64, 36000, 64, w.q_lens)
    assert need > kb.KVATTN_NOALLOC_SCRATCH_BYTES
    ref_ws = c.forward(mirror=True)
    out = torch.full_like(c.q, float("nan"))
    torch.cuda.synchronize()
    c.pool.forward_noalloc(w.layer, c.q, c.tables, c.ctx, c.ql, 36000, 64, out, scale=w.scale,
                           q_lens_host=w.q_lens)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), bits(ref_ws))
    rows = [0, 17, 40, 63]
    ref = c.oracle()  # one sequence: the oracle over its 64 rows
    assert_close(out_f64(out)[rows], ref[rows], wl.I8, w.name)


def test_noalloc_refuses_oversize_call():
    """A call whose plan needs more than the static scratch is refused before any launch."""
    announce("noalloc oversize refusal")
    w = wl.make("noalloc_tiny", seed=230, dtype=wl.BF16, num_seqs_ctx=[64], q_lens=[1],
                num_q_heads=32, num_kv_heads=8, head_dim=128)
    c = DeviceCase(w)
    # bounds alone (no host mirror): 2048 split-K tokens x 32 q-heads x 128 splits of 130 floats
    max_ctx = 262144
    need = kb.kvattn_workspace_size(c.pool.handle, 32, 1, 2048, max_ctx, 1, None)
    assert need > kb.KVATTN_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(2048, 32, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.zeros_like(q)
    tables = torch.zeros(1, max_ctx // 16, dtype=torch.int32, device="cuda")
    with pytest.raises(kb.KVPoolError) as e:
        kb.kvattn_forward_noalloc(c.pool.handle, 0, q, out, 32, 0.088, tables, tables.shape[1],
                                  c.ctx, c.ql, 1, 2048, max_ctx, 1)
    assert e.value.code == kb.KV_ENOMEM
    assert "static buffer" in str(e.value)
    torch.cuda.synchronize()
    assert int(out.abs().sum().item()) == 0  # nothing was launched
