"""The contiguous pool allocator (rssm_pool.h) on the GPU.

A torch process can install it only before its first device allocation, so
the torch-level check runs in a child process: with every allocation routed
through rssm_torch_pool_alloc, a small materialize and a small decode step
still match the oracle."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import numpy as np, torch
import replayssm_persistent_rssm_amd as rp
rp.use_contiguous_allocator()
import parity, oracle
import rssm_harness as hx, rssm_inputs as ri
dev = torch.device("cuda:0")
prob = ri.make_problem(ri.CONFIGS["tiny_f32"], 1000)
dp = hx.upload(prob, dev)
hx.materialize(dp, hx.tables(dp, dev))
torch.cuda.synchronize()
parity.check_against_oracle(prob, hx.download(dp.state, prob.state), None)
sp = ri.make_ssu_problem(ri.SSU_CONFIGS["ssu_small"], 15)
sd = ri.ssu_to_device(sp, dev)
hx.ssu_call(sd)
torch.cuda.synchronize()
_, _, _, y_g = hx.ssu_download(sd)
_, _, _, y, ym, _ = oracle.ssu_decode(sp)
live = sp.slots != -1
assert (np.abs(y_g[live] - y[live]) <= 2e-5 * ym[live]).all()
print("child ok", flush=True)
'''


def test_pool_alloc_contiguous_and_freed():
    import torch
    assert torch.cuda.is_available()
    import replayssm_persistent_rssm_amd as rp
    addr, contiguous = rp.rssm_pool_alloc(1 << 30)
    try:
        assert addr and addr % 256 == 0
        print("[gpu-pool] 1 GiB contiguous:", contiguous, flush=True)
        assert contiguous, "a 1 GiB contiguous range should be available"
    finally:
        rp.rssm_pool_free(addr)
    with pytest.raises(rp.RssmError):
        rp.rssm_pool_alloc(0)


def test_torch_allocations_through_the_pool_allocator():
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"))
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=150)
    print(res.stdout[-2000:], res.stderr[-2000:], flush=True)
    assert res.returncode == 0 and "child ok" in res.stdout
