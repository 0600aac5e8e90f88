"""Compile materialize_caller.c, a plain C program that calls
librssm_materialize through include/rssm_materialize.h and the HIP runtime
alone, with gcc.  The library must be built first (it is linked by name and
found next to the package at run time through the executable's rpath)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "replayssm_persistent_rssm_amd")
SRC = os.path.join(HERE, "materialize_caller.c")
EXE = os.path.join(HERE, "materialize_caller")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    # the HIP runtime header needs its platform macro when the compiler is not hipcc
    cmd = ["gcc", "-std=c99", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROCM, "include"), SRC,
           "-o", EXE + ".tmp", "-L" + PKG, "-lrssm_materialize", "-L" + os.path.join(ROCM, "lib"),
           "-lamdhip64", "-Wl,-rpath,$ORIGIN/../../replayssm_persistent_rssm_amd",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
