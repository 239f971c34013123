"""GPU parity of prefill with key ranges: when a call's prefill row tiles leave CUs idle, each
row tile's keys are cut into ranges reduced by separate workgroups and merged in range order
(attn_reduce_prefill).  Ranges are forced here with KVATTN_PREFILL_KSPLIT (and the workgroup plan
with KVATTN_PREFILL_WAVES / _RBLK) and compared with the oracle, including empty ranges (rows or
whole row tiles with no key in a range), half-wave pairs, int8 pools and the automatic choice.
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


# prefill chunks over short and long prefixes beside decode and verification rows, ragged
CASES = {
    "chunks": dict(num_seqs_ctx=[1900, 700, 5000, 96, 2600], q_lens=[300, 1, 200, 96, 4]),
    "one_chunk": dict(num_seqs_ctx=[4096 + 512], q_lens=[512]),
    "short": dict(num_seqs_ctx=[223, 218, 40, 300, 70], q_lens=[200, 200, 33, 290, 70]),
}


def run_case(name, dtype, ks, plan=None, monkeypatch=None, seed=501, mirror=True):
    monkeypatch.setenv("KVATTN_PREFILL_KSPLIT", str(ks))
    if plan:
        w_, _, r_ = plan.partition(":")
        monkeypatch.setenv("KVATTN_PREFILL_WAVES", w_)
        if r_:
            monkeypatch.setenv("KVATTN_PREFILL_RBLK", r_)
    announce(f"prefill ranges {name} {dtype} ks={ks} plan={plan}")
    cfg = CASES[name]
    w = wl.make(f"pfr_{name}_{dtype}_{ks}", seed=seed, dtype=dtype, num_q_heads=40, num_kv_heads=8,
                head_dim=128, **cfg)
    c = DeviceCase(w)
    c.append()
    out = c.forward(mirror=mirror)
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle(), dtype, w.name, q_lens=w.q_lens)
    return c, out


@pytest.mark.parametrize("ks", [2, 3, 5, 8])
@pytest.mark.parametrize("name", sorted(CASES))
def test_ranges_bf16(name, ks, monkeypatch):
    run_case(name, wl.BF16, ks, monkeypatch=monkeypatch)


@pytest.mark.parametrize("plan", ["8:4", "12:10", "6:3", "4"])
def test_ranges_with_half_pairs(plan, monkeypatch):
    run_case("short", wl.BF16, 3, plan=plan, monkeypatch=monkeypatch)
    run_case("chunks", wl.BF16, 4, plan=plan, monkeypatch=monkeypatch, seed=502)


@pytest.mark.parametrize("ks", [2, 6])
def test_ranges_int8(ks, monkeypatch):
    run_case("chunks", wl.I8, ks, monkeypatch=monkeypatch)


def test_ranges_without_mirror(monkeypatch):
    """Grids and workspace sized from the bounds (no host q_lens)."""
    run_case("chunks", wl.BF16, 3, monkeypatch=monkeypatch, mirror=False)


def test_ranges_reproducible(monkeypatch):
    """The same call twice gives the same bits (the ranges merge in a fixed order)."""
    c, out = run_case("one_chunk", wl.BF16, 5, monkeypatch=monkeypatch)
    again = c.forward(mirror=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), bits(again))


def test_automatic_choice(monkeypatch):
    """No override: the library picks the ranges for a chunk that leaves CUs idle."""
    monkeypatch.delenv("KVATTN_PREFILL_KSPLIT", raising=False)
    announce("prefill ranges automatic")
    w = wl.make("pfr_auto", seed=503, dtype=wl.BF16, num_q_heads=40, num_kv_heads=8, head_dim=128,
                **CASES["one_chunk"])
    c = DeviceCase(w)
    c.append()
    out = c.forward(mirror=True)
    torch.cuda.synchronize()
    assert_close(out_f64(out), c.oracle(), wl.BF16, w.name, q_lens=w.q_lens)
