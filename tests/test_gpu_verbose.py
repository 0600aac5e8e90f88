"""RSSM_MATERIALIZE_VERBOSE: with the variable set, each launch prints one
line naming the instance and its launch shape on stderr; unset (or "0"),
nothing.  The library reads the variable once per process, so each setting
runs in a child process of its own (the pull-request page's review of the
operation singles out the verbose switch and its per-call environment read)."""
import os
import re
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import torch
import parity
import rssm_harness as hx, rssm_inputs as ri
dev = torch.device("cuda:0")
prob = ri.make_problem(ri.CONFIGS["tiny_f32"], 1000)
dp = hx.upload(prob, dev)
for _ in range(2):
    hx.materialize(dp, hx.tables(dp, dev))
torch.cuda.synchronize()
parity.check_against_oracle(prob, hx.download(dp.state, prob.state), None)
print("child ok", flush=True)
'''


def _run(value):
    env = dict(os.environ)
    env.pop("RSSM_MATERIALIZE_VERBOSE", None)
    if value is not None:
        env["RSSM_MATERIALIZE_VERBOSE"] = value
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"))
    print(f"[gpu-verbose] child with RSSM_MATERIALIZE_VERBOSE={value!r}", flush=True)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=150, env=env)
    print(res.stdout[-1000:], res.stderr[-2000:], flush=True)
    assert res.returncode == 0 and "child ok" in res.stdout
    return [ln for ln in res.stderr.splitlines() if ln.startswith("[rssm_")]


def test_verbose_prints_one_line_per_launch():
    lines = _run("1")
    assert len(lines) == 2, lines
    pat = re.compile(r"^\[rssm_materialize\] materialize<kF32,kF32,16x16,kmax8,sr0> grid=(\d+) block=256 lds=\d+B "
                     r"L=1 B=2 H=4 checkpoints=1$")
    for ln in lines:
        m = pat.match(ln)
        assert m, ln
        assert int(m.group(1)) > 0


@pytest.mark.parametrize("value", [None, "0"])
def test_quiet_without_verbose(value):
    assert _run(value) == []


def _launch_config(**kw):
    import replayssm_persistent_rssm_amd as rp
    base = dict(num_layers=2, batch=4, num_heads=8, heads_per_group=1, dim=64, dstate=128, max_window=16,
                ring_buffer_len=16, input_dtype="bf16")
    base.update(kw)
    return rp.rssm_materialize_launch_config(**base)


@pytest.mark.parametrize("state_dtype", ["i8", "f8e4m3"])
def test_launch_config_grid_rule(state_dtype):
    """Default grid: the instance's resident capacity (a whole multiple of the
    compute units), eight times it for one-byte state with stochastic
    rounding (a separate instance, whose resident capacity is again a
    multiple of the compute units); max_workgroups replaces either."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    g0, b0, s0 = _launch_config(state_dtype=state_dtype, philox_rounds=0)
    g1, b1, s1 = _launch_config(state_dtype=state_dtype, philox_rounds=10)
    print(f"[gpu-launch] {state_dtype}: rne grid {g0}, sr grid {g1}, cus {cus}", flush=True)
    assert g0 > 0 and g0 % cus == 0
    assert b1 == b0 == 256 and g1 % 8 == 0 and (g1 // 8) % cus == 0
    assert _launch_config(state_dtype=state_dtype, philox_rounds=10, max_workgroups=37)[0] == 37
    assert _launch_config(state_dtype=state_dtype, philox_rounds=0, max_workgroups=37)[0] == 37
    gb = _launch_config(state_dtype="bf16")[0]
    assert gb > 0 and gb % cus == 0
