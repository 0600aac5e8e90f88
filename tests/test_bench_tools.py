"""Host-side helpers of bench.py (no GPU): the kernel source hash that keys the
committed counter summaries, the stale-summary rule behind roofline.traffic,
and the rocprofv3 stats summary format."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_code_only_ignores_comments_and_layout():
    a = "int f(int x) {  // add one\n  return x + 1; /* block\n comment */ }\n"
    b = "int f(int x)\n{\n\treturn x + 1;\n}"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(a.replace("x + 1", "x + 2"))


def test_kernel_hash_follows_code_not_comments(tmp_path, monkeypatch):
    src = tmp_path / "k.h"
    src.write_text("__device__ int g(int v) { return v * 3; }  // triple\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_hash(["k.h"])
    src.write_text("// a new comment\n__device__ int g(int v)\n{ return v * 3; }\n")
    assert bench.kernel_hash(["k.h"]) == h0
    src.write_text("__device__ int g(int v) { return v * 4; }\n")
    assert bench.kernel_hash(["k.h"]) != h0


def test_counter_summary_from_other_code_gives_no_traffic(tmp_path, monkeypatch):
    """roofline.traffic is null unless the committed summary was taken on the
    current kernel code (its kernel_source_hash line matches)."""
    (tmp_path / "profiles").mkdir()
    (tmp_path / "k.h").write_text("__global__ void k() {}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setitem(bench.COUNTER_SOURCES, "large_bf16", ["k.h"])
    summary = tmp_path / "profiles" / bench.COUNTER_FILE["large_bf16"]
    body = "# comment: not a value\nhbm_bytes_per_launch: 1234\ntraffic_over_algorithmic: 1.0001\n"
    summary.write_text(f"kernel_source_hash: {bench.kernel_hash(['k.h'])}\n" + body)
    assert bench.traffic_from_profile("large_bf16") == 1234
    assert bench.traffic_ratio("large_bf16") == pytest.approx(1.0001)
    summary.write_text("kernel_source_hash: 0000000000000000\n" + body)
    assert bench.traffic_from_profile("large_bf16") is None
    assert bench.traffic_ratio("large_bf16") is None
    summary.unlink()
    assert bench.traffic_from_profile("large_bf16") is None


def test_committed_counter_summary_is_stale_for_current_kernel():
    """The committed large_bf16 counter summary predates the current kernel
    source, so the bench line must report no traffic figure from it."""
    assert bench.traffic_from_profile("large_bf16") is None


def test_trace_summary_format(tmp_path):
    csv = tmp_path / "kt_kernel_stats.csv"
    csv.write_text('"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
                   '"void rssm::materialize_kernel<1>(rssm::KernelArgs)",11,188751939,17159267.18,70.37,17106101,17352950,0\n')
    out = bench.trace_summary(str(csv)).splitlines()
    assert out[0].startswith("# rocprofv3 kernel stats (ns)")
    assert out[1] == ("void rssm::materialize_kernel<1>(rssm::KernelArgs) | 11 | 17159267 | 17106101 | 17352950 | "
                      "188751939 | 70.37")


def test_more_than_one_gpu_is_refused():
    import subprocess
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2 and "one GPU" in res.stderr
