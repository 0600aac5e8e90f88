"""The C ABI on its own: plain C programs (tests/c_caller/materialize_caller.c
for rssm_materialize and rssm_materialize_checkpoints, step_caller.c for
rssm_ssu_decode and rssm_gdn_commit) call librssm_materialize through
include/*.h and the HIP runtime, with no Python and no torch in their
process.  The GPU cases hand them seeded problems as raw files and compare
what they write back with the CPU oracle, with the comparisons of the other
parity tests.  The CPU cases check how they link and that their host checks
refuse out-of-range slots before any HIP call.
"""
import glob
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import rssm_inputs as ri

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CALLER_DIR = os.path.join(ROOT, "tests", "c_caller")


def say(*a):
    print("[c-caller]", *a, flush=True)
    sys.stdout.flush()


def _builder():
    sys.path.insert(0, CALLER_DIR)
    try:
        import build_caller
    finally:
        sys.path.remove(CALLER_DIR)
    if not (os.path.exists(build_caller.EXE) and os.path.exists(build_caller.STEP_EXE)):
        build_caller.build()     # gcc, about a second; build() of the repository builds them too
    return build_caller


def caller_exe() -> str:
    return _builder().EXE


def step_exe() -> str:
    return _builder().STEP_EXE


def write_problem(prob, d, max_workgroups=0, checkpoints=None):
    """Raw files of one problem in the layout the caller reads; checkpoints =
    (dst [C][L][B], prefix [C][B]) makes it a multi-checkpoint call."""
    s, m = prob.spec, prob.meta
    has_scale = prob.scale is not None
    has_seed = s.philox_rounds > 0
    head = [s.L, s.B, s.H, s.hpg, s.dim, s.dstate, s.W, s.R, s.pad_slot_id, s.philox_rounds,
            ri.DTYPE_CODE[s.state_dtype], ri.DTYPE_CODE[s.input_dtype], max_workgroups, int(has_scale),
            int(has_seed), 0 if checkpoints is None else int(checkpoints[0].shape[0])]
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
    dst, pre = (m.dst, m.prefix) if checkpoints is None else checkpoints
    for name, a in (("src", m.src), ("dst", dst), ("ring_start", m.ring_start), ("prefix", pre),
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


def run_step(op, d, timeout=120):
    return subprocess.run([step_exe(), op, str(d)], capture_output=True, text=True, timeout=timeout)


def _write_fields(d, desc, tensors):
    with open(os.path.join(d, "desc.txt"), "w") as f:
        f.write("".join(f"{k} {int(v)}\n" for k, v in desc.items()))
    for name, a in tensors.items():
        if a is not None:
            np.ascontiguousarray(a).tofile(os.path.join(d, name + ".bin"))


def write_ssu(prob, d, max_workgroups=0):
    """Raw files of a decode-step problem for `step_caller ssu`; y starts as NaN."""
    s, pl = prob.spec, prob.pools
    state, xr, Br, dtr = pl.state[0], pl.x[0], pl.Bm[0], pl.dt[0]
    desc = dict(batch=s.B, num_heads=s.H, heads_per_group=s.hpg, dim=s.dim, dstate=s.dstate,
                ring_buffer_len=s.R, tokens=s.T, num_slots=state.shape[0], pad_slot_id=s.pad_slot_id,
                state_dtype=ri.DTYPE_CODE[s.state_dtype], input_dtype=ri.DTYPE_CODE[s.input_dtype],
                dt_softplus=int(s.dt_softplus), max_workgroups=max_workgroups,
                state_slot_stride=state.shape[1], x_slot_stride=xr.shape[1], B_slot_stride=Br.shape[1],
                dt_slot_stride=dtr.shape[1])
    y = np.full((s.B, s.T, s.H, s.dim), np.nan, np.float32)
    _write_fields(d, desc, dict(state=state, x_ring=xr, B_ring=Br, dt_ring=dtr, A=prob.A, D=prob.D,
                                dt_bias=prob.dt_bias, x_new=prob.x_new, B_new=prob.B_new, C_new=prob.C_new,
                                dt_new=prob.dt_new, z=prob.z, y=y, slots=prob.slots.astype(np.int32),
                                ring_start=prob.ring_start.astype(np.int32),
                                num_buffered=prob.num_buffered.astype(np.int32)))


def read_ssu(prob, d):
    pl = prob.pools
    rd = lambda name, like: np.fromfile(os.path.join(d, name + ".out"), like.dtype).reshape(like.shape)  # noqa: E731
    y = np.fromfile(os.path.join(d, "y.out"), np.float32).reshape(prob.spec.B, prob.spec.T, prob.spec.H,
                                                                   prob.spec.dim)
    return rd("x_ring", pl.x[0]), rd("B_ring", pl.Bm[0]), rd("dt_ring", pl.dt[0]), y


def write_gdn(prob, d, max_workgroups=0):
    """Raw files of a commit problem for `step_caller gdn`."""
    s = prob.spec
    desc = dict(num_layers=s.L, slots=s.slots, num_v_heads=s.HV, num_k_heads=s.H, window=s.T, batch=s.B,
                use_l2norm=int(s.use_l2norm), null_block_id=s.null_block_id, max_workgroups=max_workgroups)
    i32 = lambda a: None if a is None else np.asarray(a, np.int32)  # noqa: E731
    _write_fields(d, desc, dict(checkpoint_state=prob.state, rawv_cache=prob.rawv, rawk_cache=prob.rawk,
                                g_cache=prob.g, beta_cache=prob.beta, state_indices=i32(prob.state_indices),
                                accept_lens=i32(prob.accept_lens),
                                track_state_indices=i32(prob.track_state_indices),
                                track_steps=i32(prob.track_steps)))


# --------------------------------------------------------------------------
# CPU: linkage and host checks
# --------------------------------------------------------------------------
@pytest.mark.parametrize("which", ["materialize", "step"])
def test_caller_links_only_the_library_and_the_hip_runtime(which):
    exe = caller_exe() if which == "materialize" else step_exe()
    needed = subprocess.run(["readelf", "-d", exe], capture_output=True, text=True, check=True).stdout
    libs = set(re.findall(r"\(NEEDED\).*\[(.+?)\]", needed))
    assert "librssm_materialize.so" in libs
    assert not [x for x in libs if "torch" in x or "python" in x], libs
    undef = subprocess.run(["nm", "-D", "--undefined-only", exe], capture_output=True, text=True,
                           check=True).stdout
    used = set(re.findall(r"\b(rssm_\w+)", undef))
    declared = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        declared |= set(re.findall(r"\b(rssm_\w+)\s*\(", open(h).read()))
    want = {"materialize": {"rssm_materialize", "rssm_materialize_checkpoints"},
            "step": {"rssm_ssu_decode", "rssm_gdn_commit"}}[which]
    assert want <= used <= declared, (used, declared)


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


def test_step_caller_refuses_out_of_range_metadata(tmp_path):
    """Decode step: a live slot past the pool; commit: an accepted count past
    the window.  Both are refused before any HIP call."""
    prob = ri.make_ssu_problem(ri.SSU_CONFIGS["ssu_small"], 40)
    b = int(np.flatnonzero(prob.slots != prob.spec.pad_slot_id)[0])
    prob.slots[b] = prob.pools.state[0].shape[0]
    (tmp_path / "ssu_bad_slot").mkdir()
    write_ssu(prob, tmp_path / "ssu_bad_slot")
    res = run_step("ssu", tmp_path / "ssu_bad_slot", timeout=60)
    assert res.returncode == 1 and "outside the pool" in res.stderr, (res.returncode, res.stderr)
    g = ri.make_gdn_problem(ri.GDN_CONFIGS["gdn_small"], 41)
    g.accept_lens[0] = g.spec.T + 1
    (tmp_path / "gdn_bad_accept").mkdir()
    write_gdn(g, tmp_path / "gdn_bad_accept")
    res = run_step("gdn", tmp_path / "gdn_bad_accept", timeout=60)
    assert res.returncode == 1 and "accept_lens" in res.stderr, (res.returncode, res.stderr)
    os.remove(tmp_path / "gdn_bad_accept" / "rawk_cache.bin")
    res = run_step("gdn", tmp_path / "gdn_bad_accept", timeout=60)
    assert res.returncode == 1 and "cannot open" in res.stderr, (res.returncode, res.stderr)
    # a track slot that is another request's live state slot
    g = ri.make_gdn_problem(ri.GDN_CONFIGS["gdn_small"], 42)
    live = [b for b in range(g.spec.B) if g.state_indices[b] > g.spec.null_block_id]
    assert g.track_state_indices is not None and len(live) >= 2
    g.track_state_indices[live[0]] = g.state_indices[live[1]]
    (tmp_path / "gdn_bad_track").mkdir()
    write_gdn(g, tmp_path / "gdn_bad_track")
    res = run_step("gdn", tmp_path / "gdn_bad_track", timeout=60)
    assert res.returncode == 1 and "track slot" in res.stderr, (res.returncode, res.stderr)
    # a decode-step tensor of the wrong size
    (tmp_path / "ssu_bad_size").mkdir()
    prob = ri.make_ssu_problem(ri.SSU_CONFIGS["ssu_small"], 43)
    write_ssu(prob, tmp_path / "ssu_bad_size")
    np.zeros(3, np.float32).tofile(tmp_path / "ssu_bad_size" / "A.bin")
    res = run_step("ssu", tmp_path / "ssu_bad_size", timeout=60)
    assert res.returncode == 1 and "the shapes give" in res.stderr, (res.returncode, res.stderr)


# --------------------------------------------------------------------------
# GPU: the callers' results against the oracle
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


@pytest.mark.gpu
@pytest.mark.parametrize("state,rounds", [("bf16", 0), ("i8", 0), ("f8e4m3", 10)])
def test_checkpoints_caller_matches_the_oracle(tmp_path, state, rounds):
    """Two checkpoints per request, the first an in-place flush."""
    import parity
    spec = ri.Spec("c_ck_" + state, L=2, B=4, H=8, hpg=4, dim=64, dstate=128, R=8, W=8, state_dtype=state,
                   input_dtype="bf16", slots=12, slot_mode="perm", philox_rounds=rounds,
                   rand_seed=55 if rounds else None)
    prob = ri.make_problem(spec, 50)
    dst, pre = ri.make_checkpoints(spec, prob.meta, 51, 2, in_place=True)
    say("checkpoints", state, rounds, "dst", dst.tolist(), "prefix", pre.tolist())
    write_problem(prob, tmp_path, checkpoints=(dst, pre))
    res = run_caller(tmp_path)
    say(res.stdout.strip().replace("\n", " | "))
    assert res.returncode == 0, (res.returncode, res.stdout, res.stderr)
    st, sc = read_result(prob, tmp_path)
    parity.check_checkpoints_against_oracle(prob, dst, pre, st, sc)


@pytest.mark.gpu
@pytest.mark.parametrize("seed,wg", [(60, 0), (61, 3)])
def test_step_caller_decode_matches_the_oracle(tmp_path, seed, wg):
    import test_gpu_ssu
    prob = ri.make_ssu_problem(ri.SSU_CONFIGS["ssu_small"], seed)
    say("ssu_small seed", seed, "max_workgroups", wg, "slots", prob.slots.tolist())
    write_ssu(prob, tmp_path, max_workgroups=wg)
    res = run_step("ssu", tmp_path)
    assert res.returncode == 0, (res.returncode, res.stdout, res.stderr)
    test_gpu_ssu.check(prob, read_ssu(prob, tmp_path), f"C caller ssu_small/{seed}")


@pytest.mark.gpu
@pytest.mark.parametrize("seed,wg", [(62, 0), (63, 5)])
def test_step_caller_commit_matches_the_oracle(tmp_path, seed, wg):
    import test_gpu_gdn
    prob = ri.make_gdn_problem(ri.GDN_CONFIGS["gdn_small"], seed)
    say("gdn_small seed", seed, "max_workgroups", wg, "accept", prob.accept_lens.tolist())
    write_gdn(prob, tmp_path, max_workgroups=wg)
    res = run_step("gdn", tmp_path)
    assert res.returncode == 0, (res.returncode, res.stdout, res.stderr)
    got = np.fromfile(tmp_path / "checkpoint_state.out", np.float32).reshape(prob.state.shape)
    w = test_gpu_gdn.check(prob, got, f"C caller gdn_small/{seed}")
    assert w.any()


@pytest.mark.gpu
def test_empty_call_cost_from_c(tmp_path):
    """A call whose active list is empty, made back to back from C (no
    Python): the pages' no-write case.  The bf16 64x128 instance at its
    default grid (the resident capacity), as in the large workloads; the
    cost must stay within 5 us per call."""
    prob = ri.make_problem(ri.CONFIGS["mid_bf16"], 1001)
    write_problem(prob, tmp_path)
    res = subprocess.run([caller_exe(), str(tmp_path), "2000"], capture_output=True, text=True, timeout=120)
    say(res.stdout.strip().replace("\n", " | "))
    assert res.returncode == 0, (res.returncode, res.stdout, res.stderr)
    us = float(re.search(r"empty_call_us ([0-9.]+)", res.stdout).group(1))
    grid = int(re.search(r"launch grid=(\d+)", res.stdout).group(1))
    say("empty call from C:", us, "us per call at grid", grid)
    assert us <= 5.0, us
