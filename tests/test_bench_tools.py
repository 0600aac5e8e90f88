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


@pytest.mark.parametrize("workload", sorted(bench.COUNTER_FILE))
def test_committed_counter_summaries_follow_the_hash_rule(workload):
    """Each committed counter summary gives a traffic figure exactly when it
    was taken on the current kernel source; such a figure is the algorithmic
    bytes plus at most a few percent (re-reads, partial lines)."""
    path = os.path.join(ROOT, "profiles", bench.COUNTER_FILE[workload])
    assert os.path.exists(path), path
    lines = [ln for ln in open(path) if ln.startswith("kernel_source_hash:")]
    assert len(lines) == 1
    current = lines[0].split(":", 1)[1].strip() == bench.kernel_hash(bench.COUNTER_SOURCES[workload])
    ratio = bench.traffic_ratio(workload)
    if not current:
        assert ratio is None and bench.traffic_from_profile(workload) is None
        return
    assert 1.0 <= ratio < 1.1
    vals = bench.counter_values(workload)
    assert float(vals["hbm_bytes_per_launch"]) == pytest.approx(ratio * float(vals["algorithmic_bytes_per_launch"]),
                                                                rel=1e-3)


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


def test_valu_summary_row(tmp_path):
    """The vector-ALU row: the last dispatch of the named kernel, its counters,
    valu_time = instructions x 4 cycles / 1024 SIMDs / 2.4 GHz, and
    instructions x 64 lanes / elements."""
    csv = tmp_path / "valu_counter_collection.csv"
    rows = ['"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"']
    for d, ins in ((1, 100.0), (2, 2.4e9)):
        for c, v in (("SQ_INSTS_VALU", ins), ("SQ_ACTIVE_INST_VALU", ins * 1.01), ("SQ_WAVES", 4096.0),
                     ("GRBM_GUI_ACTIVE", 4.0e7)):
            rows.append(f'{d},"void rssm::materialize_kernel<1>(rssm::KernelArgs)","{c}",{v}')
    rows.append('3,"__amd_rocclr_copyBuffer","SQ_INSTS_VALU",5')
    csv.write_text("\n".join(rows) + "\n")
    js = tmp_path / "bench.json"
    js.write_text('[bench] a log line\n{"valu_workload": "large_bf16", "valu_kernel": "materialize_kernel", '
                  '"valu_elements": 1600000000}\n')
    cells = [c.strip() for c in bench.valu_summary(str(csv), str(js)).split("|")]
    assert cells[0] == "large_bf16" and cells[1] == "materialize_kernel" and cells[2] == "4096"
    assert float(cells[3]) == pytest.approx(2.4e9)
    assert float(cells[6]) == pytest.approx(2.4e9 * 4 / 1024 / 2.4e9 * 1e3, rel=1e-3)
    assert int(cells[7]) == 1600000000
    assert float(cells[8]) == pytest.approx(2.4e9 * 64 / 1.6e9, abs=0.01)


def test_valu_instructions_follow_the_hash_rule(tmp_path, monkeypatch):
    """The vector-ALU figure of a materialize workload comes from the committed
    table only while its kernel_source_hash line matches the current source."""
    (tmp_path / "profiles").mkdir()
    (tmp_path / "k.h").write_text("__global__ void k() {}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setitem(bench.COUNTER_SOURCES, "large_bf16", ["k.h"])
    table = tmp_path / "profiles" / bench.VALU_FILE
    rows = ("# header\n" + bench.VALU_HEADER + "\n"
            "large_i8 | materialize_kernel | 4096 | 6.1679e+08 | 6.2e+08 | 3.5e+07 | 1.004 | 6442450944 | 6.13\n")
    table.write_text(f"kernel_source_hash (materialize): {bench.kernel_hash(['k.h'])}\n" + rows)
    assert bench.valu_instructions("large_i8") == pytest.approx(6.1679e8)
    assert bench.valu_instructions("large_f8sr") is None          # no row
    assert bench.valu_instructions("gdn_large") is None           # not a materialize workload
    table.write_text("kernel_source_hash (materialize): 0000000000000000\n" + rows)
    assert bench.valu_instructions("large_i8") is None
