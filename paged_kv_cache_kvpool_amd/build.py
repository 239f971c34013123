"""Builds libkvpool.so in-tree with hipcc for gfx950 (no torch extension machinery).

    python -m paged_kv_cache_kvpool_amd.build

Objects go to ``_build/`` at the repository root; the library lands next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libkvpool.so")
ARCH = os.environ.get("KVPOOL_ARCH", "gfx950")

SOURCES = ["kvpool.cpp", "kv_append.hip", "attn_split_mfma.hip", "attn_vec.hip",
           "attn_reduce.hip", "attn_prefill_mfma.hip", "kv_dequant.hip", "kv_host.hip"]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-I" + os.path.join(ROOT, "include"),
    # Packed fp32 (v_pk_*_f32) stays off: plain fp32 code only.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libkvpool.so)")


def _compile(src: str, csrc: str = CSRC, obj_dir: str = OBJ, extra=()) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = [_hipcc(), "-x", "hip", "-c", os.path.join(csrc, src), "-o", obj] + FLAGS + list(extra)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, csrc: str = CSRC, out: str = LIB, obj_dir: str = OBJ,
          extra=()) -> str:
    """Compile every source in `csrc` and link `out` (defaults: this package, in place)."""
    os.makedirs(obj_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda f: _compile(f, csrc, obj_dir, extra), SOURCES))
    tmp = out + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
