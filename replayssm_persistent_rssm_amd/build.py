"""Build librssm_materialize.so (the operation) and librssm_pool.so (the
contiguous-pool placement helper, a separate library so that the operation's
library exports nothing that allocates) for gfx950 with hipcc, in-tree, no JIT.

Each state dtype's kernel instances live in their own translation unit and
compile in parallel; the host launcher is one more.  Flags: -O3, C++17,
packed-fp32 instructions disabled (plain fp32 VALU code only), correctly
rounded fp32 division and square root (hipcc's default, never relaxed: the
one-byte encode divides).
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "librssm_materialize.so")
POOL_LIB_PATH = os.path.join(PKG, "librssm_pool.so")
BUILD_DIR = os.path.join(PKG, "_build")

SOURCES = ["rssm_inst_f32.hip", "rssm_inst_bf16.hip", "rssm_inst_f16.hip", "rssm_inst_i8.hip",
           "rssm_inst_f8.hip", "rssm_inst_gdn.hip", "rssm_inst_ssu.hip", "rssm_materialize.hip"]
POOL_SOURCES = ["rssm_pool.hip"]
ARCH = os.environ.get("RSSM_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I" + INCLUDE, "-I" + CSRC]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + CFLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device feature flag: drop that warning only
    noise = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(noise))
    if noise and verbose:
        print("\n".join(noise), file=sys.stderr)
    return obj


def _link(objs, path: str, verbose: bool) -> None:
    tmp = path + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(path)} failed:\n" + res.stderr)
    os.replace(tmp, path)


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile and link both libraries; returns the operation library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + POOL_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(jobs, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    _link(objs[:len(SOURCES)], LIB_PATH, verbose)
    _link(objs[len(SOURCES):], POOL_LIB_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
