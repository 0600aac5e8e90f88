"""Compile materialize_caller.c and step_caller.c, plain C programs that call
librssm_materialize through include/*.h and the HIP runtime alone, with gcc.  The library must be built first (it is linked by name and
found next to the package at run time through the executable's rpath)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "replayssm_persistent_rssm_amd")
SRC = os.path.join(HERE, "materialize_caller.c")
EXE = os.path.join(HERE, "materialize_caller")
STEP_SRC = os.path.join(HERE, "step_caller.c")
STEP_EXE = os.path.join(HERE, "step_caller")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _gcc(src: str, exe: str, verbose: bool) -> None:
    # the HIP runtime header needs its platform macro when the compiler is not hipcc
    cmd = ["gcc", "-std=c99", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROCM, "include"), src,
           "-o", exe + ".tmp", "-L" + PKG, "-lrssm_materialize", "-L" + os.path.join(ROCM, "lib"),
           "-lamdhip64", "-Wl,-rpath,$ORIGIN/../../replayssm_persistent_rssm_amd",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(exe + ".tmp", exe)


def build(verbose: bool = False) -> str:
    """Build both callers; returns the materialize caller's path."""
    _gcc(SRC, EXE, verbose)
    _gcc(STEP_SRC, STEP_EXE, verbose)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
