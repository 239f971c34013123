"""The parity helpers themselves (CPU): the per-vector check catches a single wrong (row,
q-head) vector that the whole-tensor bar lets through.  The planted mistake is made on the
host, in a copy of a reference output; no GPU is involved."""
import numpy as np
import pytest

pytest.importorskip("torch")

from tests.gpu_util import TOL, assert_close, row_owner, vector_errors  # noqa: E402
from paged_kv_cache_kvpool_amd import workloads as wl  # noqa: E402


def _reference(rows=32, heads=32, d=128, seed=0):
    rng = np.random.default_rng(seed)
    # outputs of near-uniform attention over ~4K keys: RMS about sqrt(e / L)
    return rng.standard_normal((rows, heads, d)) * 0.025


def test_clean_output_passes():
    ref = _reference()
    gpu = ref * (1 + 1e-3 * np.random.default_rng(1).standard_normal(ref.shape))
    assert_close(gpu, ref, wl.BF16, "clean")


def test_one_wrong_vector_fails_vector_check_only():
    ref = _reference()
    gpu = ref.copy()
    gpu[17, 5] *= 1.15  # one (row, q-head) vector 15% off
    d = gpu - ref
    rel = np.linalg.norm(d) / np.linalg.norm(ref)
    assert rel <= TOL[wl.BF16]["rel_l2"], "the tensor bar alone must not catch this case"
    worst, (r, h), _ = vector_errors(gpu, ref)
    assert (r, h) == (17, 5) and worst == pytest.approx(0.15, rel=1e-6)
    with pytest.raises(AssertionError, match="row 17, q-head 5"):
        assert_close(gpu, ref, wl.BF16, "planted", q_lens=[16, 16])


def test_row_owner():
    assert row_owner(0, [1, 4, 3]) == (0, 0)
    assert row_owner(1, [1, 4, 3]) == (1, 0)
    assert row_owner(4, [1, 4, 3]) == (1, 3)
    assert row_owner(5, [1, 4, 3]) == (2, 0)
    assert row_owner(3, [0, 2, 2]) == (2, 1)
