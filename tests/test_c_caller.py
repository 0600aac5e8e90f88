"""The C ABI on its own: a plain C program (tests/c_caller/materialize_caller.c)
calls librssm_materialize through include/rssm_materialize.h and the HIP
runtime, with no Python and no torch in its process.  The GPU cases hand it
seeded problems as raw files and compare what it writes back with the CPU
oracle, to the same bar as the other parity tests.  The CPU cases check how it
links and that its host checks refuse out-of-pool slots before any HIP call.
"""
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import rssm_inputs as ri

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CALLER_DIR = os.path.join(ROOT, "tests", "c_caller")
HEADER = os.path.join(ROOT, "include", "rssm_materialize.h")


def say(*a):
    print("[c-caller]", *a, flush=True)
    sys.stdout.flush()


def caller_exe() -> str:
    """The built caller; built here (gcc, about a second) only if absent."""
    sys.path.insert(0, CALLER_DIR)
    try:
        import build_caller
    finally:
        sys.path.remove(CALLER_DIR)
    if not os.path.exists(build_caller.EXE):
        build_caller.build()
    return build_caller.EXE


def write_problem(prob, d, max_workgroups=0):
    """Raw files of one problem in the layout the caller reads."""
    s, m = prob.spec, prob.meta
    has_scale = prob.scale is not None
    has_seed = s.philox_rounds > 0
    head = [s.L, s.B, s.H, s.hpg, s.dim, s.dstate, s.W, s.R, s.pad_slot_id, s.philox_rounds,
            ri.DTYPE_CODE[s.state_dtype], ri.DTYPE_CODE[s.input_dtype], max_workgroups, int(has_scale),
            int(has_seed)]
    lines = [" ".join(map(str, head))]
    for l in range(s.L):
        lines.append(" ".join(str(int(v)) for v in (m.state_stride[l], m.scale_stride[l] if has_scale else 1,
                                                     m.x_stride[l], m.B_stride[l], m.dt_stride[l])))
    with open(os.path.join(d, "problem.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    for l in range(s.L):
        for name, arrs in (("state", prob.state), ("x", prob.x), ("B", prob.Bm), ("dt", prob.dt),
                           ("A", prob.A)) + ((("scale", prob.scale),) if has_scale else ()):
            np.ascontiguousarray(arrs[l]).tofile(os.path.join(d, f"{name}_{l}.bin"))
    for name, a in (("src", m.src), ("dst", m.dst), ("ring_start", m.ring_start), ("prefix", m.prefix),
                    ("active", m.active)):
        np.ascontiguousarray(a, np.int32).tofile(os.path.join(d, f"{name}.bin"))
    if has_seed:
        np.array([s.rand_seed if s.rand_seed is not None else 0], np.int64).tofile(os.path.join(d, "seed.bin"))


def read_result(prob, d):
    st = [np.fromfile(os.path.join(d, f"state_{l}.out"), prob.state[l].dtype).reshape(prob.state[l].shape)
          for l in range(prob.spec.L)]
    sc = None
    if prob.scale is not None:
        sc = [np.fromfile(os.path.join(d, f"scale_{l}.out"), np.float32).reshape(prob.scale[l].shape)
              for l in range(prob.spec.L)]
    return st, sc


def run_caller(d, timeout=120):
    return subprocess.run([caller_exe(), str(d)], capture_output=True, text=True, timeout=timeout)


# --------------------------------------------------------------------------
# CPU: linkage and host checks
# --------------------------------------------------------------------------
def test_caller_links_only_the_library_and_the_hip_runtime():
    exe = caller_exe()
    needed = subprocess.run(["readelf", "-d", exe], capture_output=True, text=True, check=True).stdout
    libs = set(re.findall(r"\(NEEDED\).*\[(.+?)\]", needed))
    assert "librssm_materialize.so" in libs
    assert not [x for x in libs if "torch" in x or "python" in x], libs
    undef = subprocess.run(["nm", "-D", "--undefined-only", exe], capture_output=True, text=True,
                           check=True).stdout
    used = set(re.findall(r"\b(rssm_\w+)", undef))
    declared = set(re.findall(r"\b(rssm_\w+)\s*\(", open(HEADER).read()))
    assert used and used <= declared, used - declared


def _small_problem():
    return ri.make_problem(ri.CONFIGS["tiny_f32"], 1000)


def test_caller_refuses_a_slot_outside_its_pool(tmp_path):
    """The host check runs before any HIP call, so it needs no GPU."""
    prob = _small_problem()
    b = int(prob.meta.active[0])
    prob.meta.dst[0, b] = prob.state[0].shape[0]      # one past the pool
    write_problem(prob, tmp_path)
    res = run_caller(tmp_path, timeout=60)
    assert res.returncode == 1 and "outside its pool" in res.stderr, (res.returncode, res.stderr)


def test_caller_refuses_a_malformed_problem(tmp_path):
    prob = _small_problem()
    write_problem(prob, tmp_path)
    os.remove(os.path.join(tmp_path, "prefix.bin"))
    res = run_caller(tmp_path, timeout=60)
    assert res.returncode == 1 and "cannot open" in res.stderr, (res.returncode, res.stderr)
    (tmp_path / "problem.txt").write_text("1 2 3\n")
    res = run_caller(tmp_path, timeout=60)
    assert res.returncode == 1 and "malformed header" in res.stderr, (res.returncode, res.stderr)


# --------------------------------------------------------------------------
# GPU: the caller's results against the oracle
# --------------------------------------------------------------------------
CASES = {
    "tiny_f32": (ri.CONFIGS["tiny_f32"], 1000, 0),
    "mid_bf16": (ri.CONFIGS["mid_bf16"], 1001, 0),
    "i8_f16_in": (ri.Spec("c_i8", L=2, B=5, H=8, hpg=4, dim=64, dstate=128, R=8, W=8, state_dtype="i8",
                          input_dtype="f16", slots=12, slot_mode="perm", stride_pad="per_layer"), 31, 0),
    "f8e4m3_philox": (ri.Spec("c_f8sr", L=2, B=5, H=8, hpg=4, dim=64, dstate=128, R=8, W=8,
                              state_dtype="f8e4m3", input_dtype="bf16", slots=12, slot_mode="perm",
                              philox_rounds=10, rand_seed=4321), 32, 0),
    "bf16_philox_3_workgroups": (ri.Spec("c_bf16sr", L=3, B=6, H=8, hpg=2, dim=64, dstate=128, R=16, W=16,
                                         k_hi=16, state_dtype="bf16", input_dtype="f32", n_active=4, slots=14,
                                         slot_mode="perm", pad_frac=0.2, philox_rounds=7, rand_seed=99), 33, 3),
}


@pytest.mark.gpu
@pytest.mark.parametrize("name", list(CASES))
def test_caller_matches_the_oracle(tmp_path, name):
    import parity
    spec, seed, wg = CASES[name]
    say(name, "seed", seed, "max_workgroups", wg, spec)
    prob = ri.make_problem(spec, seed)
    write_problem(prob, tmp_path, max_workgroups=wg)
    res = run_caller(tmp_path)
    say(res.stdout.strip().replace("\n", " | "))
    assert res.returncode == 0, (res.returncode, res.stdout, res.stderr)
    m = re.search(r"launch grid=(\d+) block=(\d+) lds_bytes=(\d+)", res.stdout)
    assert m and int(m.group(1)) > 0 and int(m.group(2)) > 0
    if wg:
        assert int(m.group(1)) == wg
    assert "refused: " in res.stdout and "materialize ok" in res.stdout
    st, sc = read_result(prob, tmp_path)
    parity.check_against_oracle(prob, st, sc)
