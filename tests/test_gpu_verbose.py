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
