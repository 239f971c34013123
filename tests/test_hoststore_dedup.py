"""The host page store's dedup resolution (csrc/host_dedup.h), on the CPU: the library merges two
pages only when their bytes are equal, whatever their 128-bit hashes say.  Hashes are injected so
that they collide (all equal, or a few values for many contents); a C++ driver runs the library's
resolution with contents stood for by ids, and the result must be the byte-equality classes of
the oracle's store model (NInfer serving doc, "Server options", --kv-host-cache-mib: equal pages
stored once)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "hoststore_dedup_driver.cpp")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:  # pragma: no cover
        pytest.skip("no C++ compiler")
    exe = str(tmp_path_factory.mktemp("dedup") / "driver")
    subprocess.run([cxx, "-std=c++17", "-O1", "-Wall", "-o", exe, SRC], check=True)
    return exe


def run(exe, stored, blocks):
    """stored: [(slot, hash, content)], blocks: [(hash, content)]; hash = (a, b)."""
    lines = [str(len(stored))] + [f"{s} {h[0]} {h[1]} {c}" for s, h, c in stored]
    lines += [str(len(blocks))] + [f"{h[0]} {h[1]} {c}" for h, c in blocks]
    out = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True,
                         check=True).stdout.split("\n")
    rounds = int(out[0].split()[1])
    refs = [tuple(int(x) for x in l.split()) for l in out[1:] if l.strip()]
    return rounds, [(bool(a), b) for a, b in refs]


def check(stored, blocks, refs):
    """Every block maps to a page of its own content: a stored one if the store has that
    content, else one new page per distinct content, held by its first block."""
    slot_content = {s: c for s, _, c in stored}
    stored_contents = {c for _, _, c in stored}
    first = {}
    for j, (_, c) in enumerate(blocks):
        if c not in stored_contents:
            first.setdefault(c, j)
    for j, ((_, c), (is_stored, i)) in enumerate(zip(blocks, refs)):
        if c in stored_contents:
            assert is_stored and slot_content[i] == c, (j, c, is_stored, i)
        else:
            assert not is_stored and i == first[c], (j, c, is_stored, i)


def test_without_collisions_one_round(driver):
    rng = np.random.default_rng(0)
    contents = rng.integers(0, 40, 200)
    h = lambda c: (1000 + int(c), 7 * int(c) + 3)  # noqa: E731  (distinct contents, distinct hashes)
    stored = [(s, h(c), int(c)) for s, c in enumerate(range(0, 40, 3))]
    blocks = [(h(c), int(c)) for c in contents]
    rounds, refs = run(driver, stored, blocks)
    check(stored, blocks, refs)
    assert rounds == 1  # one compare batch settles every block


def test_all_hashes_collide(driver):
    """Every page, stored or parked, has the same hash: only bytes can tell them apart."""
    rng = np.random.default_rng(1)
    same = (0xDEADBEEF, 0x12345678)
    stored = [(s, same, int(c)) for s, c in zip([4, 9, 2], [5, 17, 11])]
    blocks = [(same, int(c)) for c in rng.integers(0, 20, 120)]
    rounds, refs = run(driver, stored, blocks)
    check(stored, blocks, refs)
    assert len({r for r in refs if not r[0]}) == len({c for _, c in blocks} - {5, 17, 11})


@pytest.mark.parametrize("seed", range(5))
def test_few_hash_values(driver, seed):
    """Many contents over a few hash values (crafted collisions), stored and new mixed."""
    rng = np.random.default_rng(10 + seed)
    hv = lambda c: (int(c) % 3, 42)  # noqa: E731
    stored_c = rng.choice(60, 12, replace=False)
    stored = [(int(s), hv(c), int(c)) for s, c in zip(rng.permutation(100)[:12], stored_c)]
    blocks = [(hv(c), int(c)) for c in rng.integers(0, 60, 300)]
    rounds, refs = run(driver, stored, blocks)
    check(stored, blocks, refs)


def test_empty_and_single(driver):
    assert run(driver, [], []) == (0, [])
    rounds, refs = run(driver, [(3, (1, 1), 7)], [((1, 1), 8)])  # hash hit, bytes differ
    assert refs == [(False, 0)]
    rounds, refs = run(driver, [(3, (1, 1), 7)], [((1, 1), 7)])
    assert refs == [(True, 3)] and rounds == 1
