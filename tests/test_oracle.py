"""The float64 oracle against its pins (CPU only)."""
import json
import os

import numpy as np
import pytest

from oracle import attention as ora
from tests import oracle_pins as pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("name,fn,kw", pins.ALL_PINS, ids=[p[0] for p in pins.ALL_PINS])
def test_pin(name, fn, kw):
    fn(**kw)


def test_split_points_from_pages():
    """Chunked prefill cut at the pages' checkpoints equals a single pass over the prompt."""
    with open(os.path.join(GOLDEN, "prefix_split_points.json")) as f:
        g = json.load(f)
    b = g["block_size"]
    assert [p // b * b for p in g["prefix_tokens"]] == g["checkpoints"]
    rng = np.random.default_rng(2048)
    cases = list(zip(g["prefix_tokens"], g["checkpoints"]))
    cases += [(1024 + t, 1024) for t in g["tail_lengths"]]
    for total, ckpt in cases:
        if total == ckpt:
            total += 16
        q = rng.standard_normal((total, 2, 8))
        k = rng.standard_normal((total, 1, 8))
        v = rng.standard_normal((total, 1, 8))
        one = ora.attention(q[ckpt:], k, v, 0.35)
        # one pass: every prompt row; keep the rows after the checkpoint
        full = ora.attention(q, k, v, 0.35)[ckpt:]
        assert np.max(np.abs(one - full)) < 1e-12, (total, ckpt)


def test_to_f64_bf16_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x7F7F, 0x3C00], np.uint16)
    got = ora.to_f64(bits, "bf16")
    assert got[0] == 1.0 and got[1] == -1.0 and got[2] == 0.0
    assert got[3] == float(np.float32(3.3895313892515355e38))
    assert got[4] == 2.0 ** -7
