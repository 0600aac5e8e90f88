"""Benchmark: ReplaySSM prefix materialize on one MI355X.

Workload (the pages' hybrid-model shape): 48 layers, physical batch 256,
256 heads per layer in 8 B groups, 64x128 state per head, bf16 state/x/B,
fp32 dt/A, 16-entry ring, max_window 8, replay_prefix_len ~ U[1, 8].
Inputs are synthetic (seeded device generator) and resident in HBM before
timing starts.  One step = one call with all 256 requests active.

Printed JSON line: "value" is the achieved algorithmic HBM throughput in GB/s
of the full-batch call (bytes the method must move -- state in and out plus
the replayed x/B/dt rows -- divided by the measured time per call).  Extra
fields: the active-count sweep {0, 1, 16, 256} (ms/call, GB/s, us/request),
the empty-launch cost (events over back-to-back calls, and graph replay), a
roofline object for the kernel, and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
WORKLOAD = "large_bf16"
SEED = 1002
SEEDS = {"large_bf16": 1002, "large_i8": 1003, "large_f8sr": 1004}
KERNEL_SOURCES = ["replayssm_persistent_rssm_amd/csrc/rssm_kernel.h",
                  "replayssm_persistent_rssm_amd/csrc/rssm_device.h"]
# Kernel sources behind each counter workload (their code hash is recorded
# with the counters, and traffic is reported only while it matches).
COUNTER_SOURCES = {
    "large_bf16": KERNEL_SOURCES, "large_i8": KERNEL_SOURCES, "large_f8sr": KERNEL_SOURCES,
    "checkpoints": KERNEL_SOURCES,
    "gdn_large": ["replayssm_persistent_rssm_amd/csrc/gdn_kernel.h", "replayssm_persistent_rssm_amd/csrc/rssm_device.h"],
    "ssu_large": ["replayssm_persistent_rssm_amd/csrc/ssu_kernel.h", "replayssm_persistent_rssm_amd/csrc/rssm_device.h"],
}
# rocprofv3 kernel-name fragment and counter-summary file of each counter workload
COUNTER_KERNEL = {"large_bf16": "materialize_kernel", "large_i8": "materialize_kernel",
                  "large_f8sr": "materialize_kernel", "checkpoints": "materialize_kernel",
                  "gdn_large": "gdn_commit_kernel", "ssu_large": "ssu_decode_kernel"}
COUNTER_FILE = {"large_bf16": "materialize_large_bf16_counters.txt",
                "large_i8": "materialize_large_i8_counters.txt",
                "large_f8sr": "materialize_large_f8sr_counters.txt",
                "checkpoints": "materialize_checkpoints_large_bf16_counters.txt",
                "gdn_large": "gdn_commit_gdn_large_counters.txt",
                "ssu_large": "ssu_decode_ssu_large_counters.txt"}


def say(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """C++ source without comments and with whitespace collapsed (the kernel
    sources hold no string literals), so that comment edits keep the hash."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_hash(sources=None) -> str:
    """Hash of a kernel's code (comments and layout ignored); default: the
    materialize kernel."""
    h = hashlib.sha256()
    for p in (sources or KERNEL_SOURCES):
        h.update(_code_only(open(os.path.join(ROOT, p)).read()).encode())
    return h.hexdigest()[:16]


def counter_values(workload: str):
    """Key/value lines of the committed counter summary of a workload, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", COUNTER_FILE[workload])
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_hash") != kernel_hash(COUNTER_SOURCES[workload]):
        return None
    return vals


def traffic_from_profile(workload: str = "large_bf16"):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel source; else None."""
    vals = counter_values(workload)
    try:
        return int(float(vals["hbm_bytes_per_launch"])) if vals else None
    except (KeyError, ValueError):
        return None


VALU_FILE = "valu_counters_by_workload.txt"
VALU_PEAK_PER_S = 1024 * 2.4e9 / 4   # wave64 VALU instructions per second: 1024 SIMDs, 4 cycles each


def valu_instructions(workload: str):
    """SQ_INSTS_VALU per call of a materialize workload from the committed
    vector-ALU table, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", VALU_FILE)
    if workload not in ("large_bf16", "large_i8", "large_f8sr") or not os.path.exists(path):
        return None
    current = None
    for line in open(path):
        if line.startswith("kernel_source_hash (materialize):"):
            current = line.split(":", 1)[1].strip() == kernel_hash(COUNTER_SOURCES["large_bf16"])
        elif current and line.startswith(workload + " |"):
            return float(line.split("|")[3])
    return None


def traffic_ratio(workload: str):
    """Counter traffic over algorithmic bytes from the committed summary (None
    if it is missing or was taken on other kernel code)."""
    vals = counter_values(workload)
    try:
        return float(vals["traffic_over_algorithmic"]) if vals else None
    except (KeyError, ValueError):
        return None


def plain_alloc_run(steps: int):
    """The headline call with torch's caching allocator (plain hipMalloc
    pools) instead of the contiguous pools, measured in a child process that
    runs before this one touches the GPU (so, on a fresh box, as the box's
    first GPU process, where plain allocations drew the slowest memory)."""
    import subprocess
    cmd = [sys.executable, os.path.abspath(__file__), "--plain-alloc", "--only-main",
           "--steps", str(steps), "--warmup", "3"]
    say("plain-allocation run in a child process:", " ".join(cmd[1:]))
    try:
        res = subprocess.run(cmd, capture_output=True, text=True, timeout=600, cwd=ROOT)
    except subprocess.TimeoutExpired:
        return {"error": "timed out"}
    for line in res.stderr.splitlines():
        if line.startswith("[bench]"):
            say("  child:", line[len("[bench] "):])
    lines = [ln for ln in res.stdout.splitlines() if ln.startswith("{")]
    if res.returncode != 0 or not lines:
        return {"error": f"exit status {res.returncode}", "stderr_tail": res.stderr[-500:]}
    r = json.loads(lines[-1])
    return {"ms_per_call": r["ms_per_step"], "GB/s": r["value"], "frac_of_hbm_peak": r["roofline"]["frac"],
            "steps": r["steps"], "pools": r["config"]["pools"],
            "note": "same workload and kernel; the pools from torch's caching allocator (hipMalloc) in a child "
                    "process run first. The headline uses physically contiguous pools (rssm_pool.h)"}


def sweep_point(dp, tabs, spec, dev, stream, n: int, reps: int):
    """(ms per call, mean algorithmic bytes) of calls with the first n entries
    of a seeded permutation of the requests active, the set rotated over up
    to 32 disjoint sets so that the 256 MB last-level cache cannot serve a
    repeated request."""
    import torch
    import rssm_harness as hx
    import rssm_inputs as ri
    perm = np.random.default_rng(SEED).permutation(spec.B).astype(np.int32)

    def active_list(ids):
        a = np.full(spec.B, -1, np.int32)
        a[:len(ids)] = ids
        return torch.from_numpy(a).to(dev)
    n_sets = 1 if n in (0, spec.B) else min(32, spec.B // n)
    ids_sets = [perm[(j * n) % spec.B:(j * n) % spec.B + n] for j in range(n_sets)]
    # one prepared call per set: the timed loop makes one C call per step
    calls_n = [hx.prepared(dp, hx.Tables(**{**tabs.__dict__, "active_request_indices": active_list(ids)}))
               for ids in ids_sets]
    it = [0]

    def rot():
        calls_n[it[0] % n_sets]()
        it[0] += 1
    # as many untimed calls as timed ones first: right after a run of lighter
    # calls (the empty ones) the first calls of a small batch run slower
    for _ in range(reps):
        rot()
    torch.cuda.synchronize()
    ms_n = timed_calls(rot, reps, stream)
    bytes_n = 0
    if n:
        tot = 0
        for ids in ids_sets:
            act = np.array([int(v) for v in ids] + [-1] * (spec.B - n), np.int32)
            tot += hx.algorithmic_bytes(spec, ri.Meta(**{**dp.meta.__dict__, "active": act}))
        bytes_n = tot // n_sets
    return ms_n, bytes_n


# active-request counts of the sweep and the calls timed at each
SWEEP = ((0, 1000), (1, 256), (16, 64), (256, 10))


def timed_calls(fn, n, stream):
    import torch
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(n):
        fn()
    stop.record(stream)
    stop.synchronize()
    return start.elapsed_time(stop) / n  # ms per call


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(dp, seconds: float):
    """The CPU oracle on a bounded sample of the same workload: the tiles of
    the first listed request, (layer, head) by (layer, head).  Timed twice:
    on one thread (the plain loop), then with one task per tile on a thread
    pool as wide as this process's CPU share (the C oracle releases the GIL),
    each for about half of `seconds`.  Only the oracle calls are timed (host
    copies of the tiles are made first)."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    import rssm_inputs as ri
    import torch
    spec, m = dp.spec, dp.meta
    b = int(m.active[0])
    n_tile = spec.dim * spec.dstate
    _, _, d_x, d_B, d_dt = ri.dense_sizes(spec)
    sb, ib = ri.ELEM_BYTES[spec.state_dtype], ri.ELEM_BYTES[spec.input_dtype]
    k, r0 = int(m.prefix[b]), int(m.ring_start[b])
    tile_bytes = (2 * spec.H * n_tile * sb + k * (spec.H * spec.dim * ib + spec.G * spec.dstate * ib + spec.H * 4)) / spec.H
    host = lambda t: (t.view(torch.int16) if t.dtype == torch.bfloat16 else t).cpu().numpy()  # noqa: E731
    layers = {}

    def layer(l):
        if l not in layers:
            s = int(m.src[l, b])
            layers[l] = (host(dp.state[l][s, :spec.H * n_tile]).view(np.uint16), host(dp.x[l][s, :d_x]).view(np.uint16),
                         host(dp.Bm[l][s, :d_B]).view(np.uint16), dp.dt[l][s, :d_dt].cpu().numpy(), dp.A[l].cpu().numpy())
        return layers[l]

    def run(unit):
        l, h = unit
        src, x, B, dt, A = layers[l]
        oracle.tile(spec, l, b, h, r0, k, float(A[h]), src[h * n_tile:(h + 1) * n_tile], None, x, B, dt)

    units = [(l, h) for l in range(spec.L) for h in range(spec.H)]
    half = seconds / 2
    # single thread: consecutive tiles until half the budget is spent
    done1, spent1 = 0, 0.0
    for l in range(spec.L):
        layer(l)
        t0 = time.perf_counter()
        for h in range(spec.H):
            run((l, h))
        spent1 += time.perf_counter() - t0
        done1 += spec.H
        if spent1 >= half:
            break
    rate1 = done1 / spent1   # tiles per second on one thread
    try:
        share = len(os.sched_getaffinity(0))
    except AttributeError:
        share = os.cpu_count() or 1
    threads = max(1, min(share, int(os.environ.get("OMP_NUM_THREADS", share)), 16))
    # all threads: the next tiles, sized to about half the budget at the ideal speed-up
    n_multi = min(len(units), max(threads * 4, int(rate1 * threads * half)))
    todo = units[done1:done1 + n_multi] if done1 + n_multi <= len(units) else units[:n_multi]
    for l in sorted(set(u[0] for u in todo)):
        layer(l)
    with ThreadPoolExecutor(max_workers=threads) as pool:
        t0 = time.perf_counter()
        list(pool.map(run, todo))
        spent_n = time.perf_counter() - t0
    rate_n = len(todo) / spent_n
    gbs = lambda tiles_per_s: round(tiles_per_s * tile_bytes / 1e9, 4)  # noqa: E731
    return {"value": gbs(rate_n), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"request {b} (k={k}), tiles of {spec.dim}x{spec.dstate} ({tile_bytes:.0f} algorithmic bytes "
                      f"each): {done1} tiles on one thread in {spent1:.1f} s, then {len(todo)} tiles on "
                      f"{threads} threads in {spent_n:.1f} s",
            "threads": threads, "host_cores": os.cpu_count(), "cpu_share": share, "cpu_model": _cpu_model(),
            "single_thread": {"value": gbs(rate1), "unit": "GB/s", "tiles": done1, "seconds": round(spent1, 2)},
            "all_threads": {"value": gbs(rate_n), "unit": "GB/s", "tiles": len(todo), "seconds": round(spent_n, 2),
                            "speedup_over_single": round(rate_n / rate1, 2)}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU oracle sample budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--only-main", action="store_true", help="profile mode: warmup + timed steps only")
    ap.add_argument("--empty-only", action="store_true", help="profile mode: 200 calls with no active request")
    ap.add_argument("--active-only", type=int, default=None, metavar="N",
                    help="profile mode: one point of the active-request sweep (N requests, rotated sets)")
    ap.add_argument("--all-pad-only", action="store_true",
                    help="profile mode: 200 calls with every request listed and every source the pad slot")
    ap.add_argument("--pmc-calibrate", action="store_true",
                    help="counter mode: 2 calls of --workload, then 2 plain device copies of 1 GiB; prints "
                         "the workload's algorithmic bytes per call as one JSON line")
    ap.add_argument("--workload", default=WORKLOAD, choices=sorted(COUNTER_KERNEL),
                    help="workload of the profile modes (the headline line always uses large_bf16); "
                         "checkpoints, gdn_large and ssu_large in --pmc-calibrate only")
    ap.add_argument("--only-gdn", action="store_true",
                    help="profile mode: the gated-delta-rule commit line only")
    ap.add_argument("--no-plain-alloc-run", action="store_true",
                    help="skip the child process that times the headline call with plain allocations")
    ap.add_argument("--plain-alloc", action="store_true",
                    help="plain hipMalloc pools (torch's caching allocator) instead of physically contiguous ones")
    ap.add_argument("--only-ssu", action="store_true",
                    help="profile mode: the decode-step line only")
    ap.add_argument("--only-checkpoints", action="store_true",
                    help="profile mode: the multi-checkpoint line of the large_bf16 workload only")
    ap.add_argument("--no-checkpoints", action="store_true",
                    help="skip the multi-checkpoint (flush + checkpoint) line")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the int8 and e4m3+Philox workload lines")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "ALG_JSON"),
                    help="print the HBM-traffic summary of two --pmc-calibrate counter runs (and the JSON "
                         "line one of them printed) and exit")
    ap.add_argument("--summarize-trace", metavar="KERNEL_STATS_CSV",
                    help="print the kernel-stats table of a --kernel-trace --stats run and exit")
    ap.add_argument("--summarize-pmc", metavar="COUNTER_CSV",
                    help="print the counter values of each materialize dispatch of a --pmc run and exit")
    ap.add_argument("--summarize-valu", nargs=2, metavar=("COUNTER_CSV", "BENCH_JSON"),
                    help="print the vector-ALU table row of a --pmc run of SQ_ACTIVE_INST_VALU, GRBM_GUI_ACTIVE, "
                         "SQ_INSTS_VALU and SQ_WAVES over --only-main/--only-gdn/--only-ssu (and the JSON line "
                         "that run printed) and exit")
    args = ap.parse_args()
    if args.summarize_pmc:
        print(pmc_summary(args.summarize_pmc), end="")
        return
    if args.summarize_valu:
        print(valu_summary(*args.summarize_valu), end="")
        return
    if args.summarize_counters:
        print(counters_summary(*args.summarize_counters), end="")
        return
    if args.summarize_trace:
        print(trace_summary(args.summarize_trace), end="")
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the path needs no collectives (each GPU would run the same kernel "
              "on its own heads, requests or layers); --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    default_run = not (args.plain_alloc or args.only_main or args.empty_only or args.all_pad_only
                       or args.active_only is not None
                       or args.pmc_calibrate or args.only_checkpoints or args.only_gdn or args.only_ssu)
    plain = plain_alloc_run(args.steps) if default_run and not args.no_plain_alloc_run else None

    import torch
    import rssm_harness as hx
    import rssm_inputs as ri
    import replayssm_persistent_rssm_amd as rp

    if not args.plain_alloc:
        # the pools physically contiguous (before the process allocates anything)
        rp.use_contiguous_allocator()
    dev = torch.device("cuda:0")
    if args.pmc_calibrate and args.workload in ("gdn_large", "ssu_large"):
        pmc_calibrate_other(args.workload, dev)
        return
    if args.workload in ("gdn_large", "ssu_large", "checkpoints") and not args.pmc_calibrate:
        raise SystemExit(f"--workload {args.workload} is a counter-mode workload (--pmc-calibrate)")
    if args.only_gdn:
        out = gdn_workload(dev, torch.cuda.current_stream(), args.steps, with_null=False)
        print(json.dumps({"gdn_commit": out, "valu_workload": "gdn_large", "valu_kernel": "gdn_commit_kernel",
                          "valu_elements": out["state_element_tokens"]}), flush=True)
        return
    if args.only_ssu:
        out = ssu_workload(dev, torch.cuda.current_stream(), args.steps)
        print(json.dumps({"ssu_decode": out, "valu_workload": "ssu_large", "valu_kernel": "ssu_decode_kernel",
                          "valu_elements": out["checkpoint_elements"]}), flush=True)
        return
    profile_mode = (args.only_main or args.empty_only or args.all_pad_only or args.pmc_calibrate
                    or args.only_checkpoints or args.active_only is not None)
    wl = args.workload if profile_mode else WORKLOAD
    if wl == "checkpoints":
        wl = "large_bf16"   # the two-checkpoint call runs on the large_bf16 problem
    spec = ri.CONFIGS[wl]
    say("generating", wl, "seed", SEEDS[wl])
    t0 = time.time()
    dp = ri.make_device_problem(spec, SEEDS[wl], dev, fill_dst=0)
    tabs = hx.tables(dp, dev)
    torch.cuda.synchronize()
    say(f"inputs resident in HBM ({time.time() - t0:.1f} s)")
    stream = torch.cuda.current_stream()
    grid, block, lds = rp.rssm_materialize_launch_config(
        num_layers=spec.L, batch=spec.B, num_heads=spec.H, heads_per_group=spec.hpg, dim=spec.dim,
        dstate=spec.dstate, max_window=spec.W, ring_buffer_len=spec.R, state_dtype=spec.state_dtype,
        input_dtype=spec.input_dtype)

    full_bytes = hx.algorithmic_bytes(spec, dp.meta)
    call = hx.prepared(dp, tabs)   # one C call per step, arguments marshalled once

    if args.only_checkpoints:
        print(json.dumps({"checkpoints": checkpoint_workload(dp, tabs, spec, stream, args.steps)}), flush=True)
        return

    if args.active_only is not None:
        n = args.active_only
        if not 0 <= n <= spec.B:
            raise SystemExit(f"--active-only must be in [0, {spec.B}]")
        reps = dict(SWEEP).get(n, 64)
        ms_n, bytes_n = sweep_point(dp, tabs, spec, dev, stream, n, reps)
        out = {"workload": wl, "active": n, "untimed_calls": reps, "timed_calls": reps,
               "ms_per_call": round(ms_n, 5), "algorithmic_bytes": bytes_n}
        if n:
            out["GB/s"] = round(bytes_n / (ms_n * 1e-3) / 1e9, 1)
        say(f"active={n}: {out}")
        print(json.dumps(out), flush=True)
        return

    if args.empty_only or args.all_pad_only or args.pmc_calibrate:
        if args.empty_only:
            empty = torch.full((spec.B,), -1, dtype=torch.int32, device=dev)
            for _ in range(200):
                call(empty)
        elif args.all_pad_only:
            pad_src = torch.full((spec.L, spec.B), spec.pad_slot_id, dtype=torch.int32, device=dev)
            pad_call = hx.prepared(dp, hx.Tables(**{**tabs.__dict__, "src_slots": pad_src}))
            for _ in range(200):
                pad_call()
        else:
            if args.workload == "checkpoints":
                dst, pre = hx.flush_and_checkpoint_tables(dp.meta)
                call = hx.prepared_checkpoints(dp, tabs, torch.from_numpy(dst).to(dev), torch.from_numpy(pre).to(dev))
                nbytes = hx.checkpoint_bytes(spec, dp.meta, dst, pre)
            else:
                nbytes = full_bytes
            for _ in range(2):
                call()
            calibration_copies(dev)
            print(json.dumps({"counter_workload": args.workload, "algorithmic_bytes": nbytes,
                              "kernel": COUNTER_KERNEL[args.workload]}), flush=True)
        torch.cuda.synchronize()
        say("done")
        return

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ms = timed_calls(call, args.steps, stream)
    torch.cuda.synchronize()
    # spread of single calls (outside the timed region)
    singles = sorted(timed_calls(call, 1, stream) for _ in range(5))
    value = full_bytes / (ms * 1e-3) / 1e9
    say(f"full batch: {ms:.3f} ms/call, {value:.1f} GB/s")
    result = {
        "metric": "materialize HBM GB/s (% of roofline) + us/request at L=48,H=256; empty-launch us",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic (seeded device generator; no dataset)",
        "config": {"workload": "large_bf16: L=48, B=256 (256 active), H=256 (8 groups), state 64x128, "
                               "bf16 state/x/B, fp32 dt/A, R=16, max_window=8, k~U[1,8]",
                   "storage": "bf16", "accumulate": "f32", "grid": grid, "block": block, "lds_bytes": lds,
                   "algorithmic_bytes_per_call": full_bytes,
                   "pools": "hipMalloc" if args.plain_alloc else "physically contiguous (rssm_pool.h)"},
        "roofline": {"bound": "hbm", "achieved": round(value, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBS, 4), "traffic": traffic_from_profile("large_bf16"),
                     "kernel": "materialize_kernel<bf16,bf16,64x128,kmax8>", "kernel_source_hash": kernel_hash()},
        "us_per_request_full": round(ms * 1e3 / spec.B, 3),
        "single_call_ms_min_med_max": [round(singles[0], 3), round(singles[2], 3), round(singles[-1], 3)],
    }
    if plain is not None:
        result["plain_alloc"] = plain
    if args.only_main:
        result.update(valu_workload=wl, valu_kernel="materialize_kernel",
                      valu_elements=written_state_elements(spec, dp.meta))
        print(json.dumps(result), flush=True)
        return

    # Practical ceilings on the same box: a plain device-to-device copy, and
    # this kernel's own zero-prefix path (pure state copy, same layout).
    a = torch.empty(4 << 30, dtype=torch.uint8, device=dev).fill_(7)
    b_ = torch.empty_like(a)
    b_.copy_(a)
    torch.cuda.synchronize()
    ms_copy = timed_calls(lambda: b_.copy_(a), 10, stream)
    del a, b_
    zero_k = torch.zeros((spec.B,), dtype=torch.int32, device=dev)
    call_k0 = hx.prepared(dp, tabs, replay_prefix_len=zero_k)
    call_k0()
    torch.cuda.synchronize()
    ms_k0 = timed_calls(call_k0, max(4, args.steps // 2), stream)
    k0_bytes = spec.L * spec.B * 2 * spec.H * spec.dim * spec.dstate * ri.ELEM_BYTES[spec.state_dtype]
    result["ceilings"] = {
        "device_copy_GB/s": round(2 * (4 << 30) / (ms_copy * 1e-3) / 1e9, 1),
        "zero_prefix_copy_GB/s": round(k0_bytes / (ms_k0 * 1e-3) / 1e9, 1),
        "note": "torch copy_ of 4 GiB (read+write bytes); the materialize kernel with every prefix 0 "
                "(state bytes in+out only)"}
    say(f"ceilings: {result['ceilings']}")

    if not args.no_sweep:
        sweep = {}
        t_empty = None
        for n, reps in SWEEP:
            ms_n, bytes_n = sweep_point(dp, tabs, spec, dev, stream, n, reps)
            if n == 0:
                t_empty = ms_n
            entry = {"ms_per_call": round(ms_n, 5), "algorithmic_bytes": bytes_n}
            if n:
                entry["GB/s"] = round(bytes_n / (ms_n * 1e-3) / 1e9, 1)
                entry["frac_of_hbm_peak"] = round(bytes_n / (ms_n * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
                entry["us_per_request"] = round(ms_n * 1e3 / n, 3)
                entry["us_per_request_slope"] = round((ms_n - t_empty) * 1e3 / n, 3)
            sweep[str(n)] = entry
            say(f"active={n}: {entry}")
        result["sweep_active"] = sweep
        result["empty_launch_us"] = round(t_empty * 1e3, 3)

        # empty launch under graph replay (100 captured calls)
        empty = torch.full((spec.B,), -1, dtype=torch.int32, device=dev)
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            hx.prepared(dp, tabs)(empty)     # warm-up on a side stream before capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            gcall = hx.prepared(dp, tabs)    # bound to the capture stream
            for _ in range(100):
                gcall(empty)
        g.replay()
        torch.cuda.synchronize()
        t_graph = timed_calls(g.replay, 10, stream) / 100
        result["empty_launch_us_graph"] = round(t_graph * 1e3, 3)
        # every request listed, every source slot the pad slot: work discovery over all
        # (request, layer) pairs, nothing written
        pad_src = torch.full((spec.L, spec.B), spec.pad_slot_id, dtype=torch.int32, device=dev)
        pad_call = hx.prepared(dp, hx.Tables(**{**tabs.__dict__, "src_slots": pad_src}))
        for _ in range(20):
            pad_call()
        torch.cuda.synchronize()
        t_pad = timed_calls(pad_call, 1000, stream)
        result["empty_launch_us_all_pad"] = round(t_pad * 1e3, 3)
        say(f"empty launch: {t_empty * 1e3:.2f} us (stream), {t_graph * 1e3:.2f} us (graph), "
            f"{t_pad * 1e3:.2f} us (all {spec.B} listed, every source the pad slot)")

    if not args.no_cpu_baseline:
        say(f"CPU oracle sample (~{args.cpu_seconds:.0f} s)")
        result["cpu_baseline"] = cpu_baseline(dp, args.cpu_seconds)

    if not args.no_checkpoints:
        result["checkpoints"] = checkpoint_workload(dp, tabs, spec, stream, max(4, args.steps // 2))

    if not args.no_other_workloads:
        del call, tabs, dp
        torch.cuda.empty_cache()
        result["other_workloads"] = {name: other_workload(name, dev, stream, max(5, args.steps // 2))
                                     for name in ("large_i8", "large_f8sr")}
        result["other_workloads"]["gdn_commit"] = gdn_workload(dev, stream, max(5, args.steps // 2))
        result["other_workloads"]["ssu_decode"] = ssu_workload(dev, stream, max(5, args.steps // 2))
    print(json.dumps(result), flush=True)


def calibration_copies(dev):
    """Two plain device copies of 1 GiB (1 GiB read and 1 GiB written each):
    the counter readings they produce scale counter KiB to bytes."""
    import torch
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    b_ = torch.empty_like(a)
    for _ in range(2):
        b_.copy_(a)
    torch.cuda.synchronize()


def pmc_calibrate_other(workload, dev):
    """Counter mode for the gated-delta-rule commit and the decode step: 2 calls
    on the full-size problem, then the calibration copies."""
    import torch
    import rssm_harness as hx
    import rssm_inputs as ri
    import replayssm_persistent_rssm_amd as rp
    if workload == "gdn_large":
        spec = ri.GDN_CONFIGS["gdn_large"]
        dp = ri.make_gdn_device_problem(spec, 1010, dev)
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)  # noqa: E731
        call = rp.GdnCommitCall(dp.state, dp.rawv, dp.rawk, dp.g, dp.beta, i32(dp.state_indices),
                                i32(dp.accept_lens), track_state_indices=i32(dp.track_state_indices),
                                track_steps=i32(dp.track_steps), null_block_id=spec.null_block_id)
        nbytes = hx.gdn_bytes(spec, dp.state_indices, dp.accept_lens, dp.track_state_indices, dp.track_steps)
    else:
        spec = ri.SSU_CONFIGS["ssu_large"]
        dp = ri.make_ssu_device_problem(spec, 1020, dev)
        call = hx.ssu_prepared(dp)
        nbytes = hx.ssu_bytes(spec, dp.slots_np, dp.num_buffered_np)
    torch.cuda.synchronize()
    for _ in range(2):
        call()
    calibration_copies(dev)
    print(json.dumps({"counter_workload": workload, "algorithmic_bytes": nbytes,
                      "kernel": COUNTER_KERNEL[workload]}), flush=True)


def checkpoint_workload(dp, tabs, spec, stream, steps):
    """The large_bf16 problem with two checkpoints per request: every buffered
    token flushed in place plus the state at half the prefix written to the
    request's destination slot -- one multi-checkpoint call, against the same
    two results from two single-checkpoint calls (checkpoint first, then the
    in-place flush).  The flush rewrites the sources, so timed calls keep
    evolving the state (values stay bounded: every token decays it)."""
    import torch
    import rssm_harness as hx
    dev = dp.state[0].device
    dst, pre = hx.flush_and_checkpoint_tables(dp.meta)
    t_dst = torch.from_numpy(dst).to(dev)
    t_pre = torch.from_numpy(pre).to(dev)
    multi = hx.prepared_checkpoints(dp, tabs, t_dst, t_pre)
    half = hx.prepared(dp, tabs, replay_prefix_len=t_pre[1])      # writes dst slots
    flush_tabs = hx.Tables(**{**tabs.__dict__, "dst_slots": t_dst[0]})
    flush = hx.prepared(dp, flush_tabs)                              # dst = src
    for _ in range(2):
        multi()
    torch.cuda.synchronize()
    ms_multi = timed_calls(multi, steps, stream)

    def two():
        half()
        flush()
    two()
    torch.cuda.synchronize()
    ms_two = timed_calls(two, steps, stream)
    nbytes = hx.checkpoint_bytes(spec, dp.meta, dst, pre)
    out = {"workload": "large_bf16 with 2 checkpoints per request: in-place flush of all k tokens + the state "
                       "after k//2 tokens in the destination slot",
           "ms_per_call": round(ms_multi, 4), "algorithmic_bytes": nbytes,
           "GB/s": round(nbytes / (ms_multi * 1e-3) / 1e9, 1),
           "frac_of_hbm_peak": round(nbytes / (ms_multi * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "two_single_calls_ms": round(ms_two, 4),
           "speedup_vs_two_calls": round(ms_two / ms_multi, 3),
           "traffic_over_algorithmic": traffic_ratio("checkpoints")}
    say(f"checkpoints: {out}")
    return out


def gdn_workload(dev, stream, steps, with_null: bool = True):
    """The gated-delta-rule commit on gdn_large: 48 layers, 256 requests (a
    sixteenth with a null slot, a sixteenth accepting nothing, the rest
    accepting U[0, 8] tokens), 32 value heads over 16 key heads, fp32 128x128
    checkpoints, 8-token bf16 windows, a tracked step per request (inside the
    prefix for about half).  The commit is in place, so timed calls keep
    evolving the states (the update never expands them)."""
    import torch
    import rssm_harness as hx
    import rssm_inputs as ri
    import replayssm_persistent_rssm_amd as rp
    spec = ri.GDN_CONFIGS["gdn_large"]
    seed = 1010
    say("generating gdn_large seed", seed)
    dp = ri.make_gdn_device_problem(spec, seed, dev)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)  # noqa: E731
    meta = [i32(dp.state_indices), i32(dp.accept_lens), i32(dp.track_state_indices), i32(dp.track_steps)]
    call = rp.GdnCommitCall(dp.state, dp.rawv, dp.rawk, dp.g, dp.beta, meta[0], meta[1],
                            track_state_indices=meta[2], track_steps=meta[3], null_block_id=spec.null_block_id)
    for _ in range(2):
        call()
    torch.cuda.synchronize()
    ms = timed_calls(call, steps, stream)
    nbytes = hx.gdn_bytes(spec, dp.state_indices, dp.accept_lens, dp.track_state_indices, dp.track_steps)
    live = int(sum(1 for b in range(spec.B) if dp.state_indices[b] > spec.null_block_id and dp.accept_lens[b] > 0))
    out = {"workload": f"gdn_large: L={spec.L}, B={spec.B} ({live} committing), HV={spec.HV}, H={spec.H}, "
                       f"fp32 128x128 K-last state, bf16 windows T={spec.T}, tracked steps",
           "ms_per_call": round(ms, 4), "algorithmic_bytes": nbytes,
           "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
           "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "us_per_request": round(ms * 1e3 / max(live, 1), 3),
           "traffic_over_algorithmic": traffic_ratio("gdn_large"),
           # state elements times the tokens each commits (the vector-ALU table's denominator)
           "state_element_tokens": sum(spec.L * spec.HV * spec.dv * spec.dk * min(int(dp.accept_lens[b]), spec.T)
                                       for b in range(spec.B)
                                       if dp.state_indices[b] > spec.null_block_id and dp.accept_lens[b] > 0)}
    # every request null: the work discovery alone (nothing is written); left
    # out in the profile mode, whose trace then holds only the full calls
    if not with_null:
        say(f"gdn_commit: {out}")
        del call, dp, meta
        torch.cuda.empty_cache()
        return out
    null_idx = torch.full((spec.B,), spec.null_block_id, dtype=torch.int32, device=dev)
    null_call = rp.GdnCommitCall(dp.state, dp.rawv, dp.rawk, dp.g, dp.beta, null_idx, meta[1],
                                 track_state_indices=meta[2], track_steps=meta[3],
                                 null_block_id=spec.null_block_id)
    for _ in range(20):
        null_call()
    torch.cuda.synchronize()
    out["all_null_us"] = round(timed_calls(null_call, 1000, stream) * 1e3, 3)
    say(f"gdn_commit: {out}")
    del call, null_call, dp, meta
    torch.cuda.empty_cache()
    return out


def ssu_workload(dev, stream, steps):
    """The decode step on ssu_large (one layer): 256 requests, 256 heads in 8
    groups, 64x128 bf16 checkpoints, bf16 inputs, ring of 16 with U[0, 12]
    pending entries, 4 new tokens per request (speculative decode), D, dt_bias
    and the z gate.  The checkpoint is read only and the append rewrites the
    same ring entries, so every timed call does identical work."""
    import torch
    import rssm_harness as hx
    import rssm_inputs as ri
    spec = ri.SSU_CONFIGS["ssu_large"]
    seed = 1020
    say("generating ssu_large seed", seed)
    dp = ri.make_ssu_device_problem(spec, seed, dev)
    call = hx.ssu_prepared(dp)
    # A call takes ~0.2 ms: measured on MI355X, the first ~60 back-to-back
    # calls of a process run up to 15% slower (the first one 1.5 ms) before
    # the time settles, so 100 untimed calls come first.
    for _ in range(100):
        call()
    torch.cuda.synchronize()
    ms = timed_calls(call, max(50, steps), stream)
    nbytes = hx.ssu_bytes(spec, dp.slots_np, dp.num_buffered_np)
    live = int((dp.slots_np != spec.pad_slot_id).sum())
    out = {"workload": f"ssu_large: B={spec.B} ({live} live), H={spec.H} (hpg {spec.hpg}), {spec.dim}x{spec.dstate} "
                       f"{spec.state_dtype} checkpoints, {spec.input_dtype} inputs, R={spec.R}, T={spec.T} new "
                       f"tokens, mean {float(dp.num_buffered_np.mean()):.2f} pending",
           "ms_per_call": round(ms, 4), "algorithmic_bytes": nbytes,
           "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
           "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "us_per_request": round(ms * 1e3 / max(live, 1), 3),
           "traffic_over_algorithmic": traffic_ratio("ssu_large"),
           "checkpoint_elements": live * spec.H * spec.dim * spec.dstate}
    say(f"ssu_decode: {out}")
    del call, dp
    torch.cuda.empty_cache()
    return out


def empty_launch_costs(dp, tabs, spec, stream):
    """Cost of a call with nothing to do, in the workload's own launch
    configuration: no active request (back-to-back calls on the stream, and
    per call under graph replay), and every request listed with every source
    slot the pad slot (back-to-back)."""
    import torch
    import rssm_harness as hx
    dev = dp.state[0].device
    empty = torch.full((spec.B,), -1, dtype=torch.int32, device=dev)
    ecall = hx.prepared(dp, hx.Tables(**{**tabs.__dict__, "active_request_indices": empty}))
    for _ in range(20):
        ecall()
    torch.cuda.synchronize()
    t_stream = timed_calls(ecall, 1000, stream)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        hx.prepared(dp, tabs)(empty)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        gcall = hx.prepared(dp, tabs)
        for _ in range(100):
            gcall(empty)
    g.replay()
    torch.cuda.synchronize()
    t_graph = timed_calls(g.replay, 10, stream) / 100
    pad_src = torch.full((spec.L, spec.B), spec.pad_slot_id, dtype=torch.int32, device=dev)
    pcall = hx.prepared(dp, hx.Tables(**{**tabs.__dict__, "src_slots": pad_src}))
    for _ in range(20):
        pcall()
    torch.cuda.synchronize()
    t_pad = timed_calls(pcall, 1000, stream)
    del g
    return {"empty_launch_us": round(t_stream * 1e3, 3), "empty_launch_us_graph": round(t_graph * 1e3, 3),
            "empty_launch_us_all_pad": round(t_pad * 1e3, 3)}


def other_workload(name, dev, stream, steps):
    """Time one call of a secondary workload (its listed requests active)."""
    import torch
    import rssm_harness as hx
    import rssm_inputs as ri
    import replayssm_persistent_rssm_amd as rp
    spec = ri.CONFIGS[name]
    say("generating", name, "seed", SEEDS[name])
    dp = ri.make_device_problem(spec, SEEDS[name], dev, fill_dst=0)
    tabs = hx.tables(dp, dev)
    call = hx.prepared(dp, tabs)
    for _ in range(20):   # the first calls of a process run slower (up to ~25% for the one-byte states)
        call()
    torch.cuda.synchronize()
    ms = timed_calls(call, steps, stream)
    nbytes = hx.algorithmic_bytes(spec, dp.meta)
    n = spec.n_active
    out = {"workload": f"L={spec.L}, B={spec.B} ({n} active), H={spec.H} (hpg {spec.hpg}), "
                       f"{spec.dim}x{spec.dstate} {spec.state_dtype} state + fp32 row scales, "
                       f"{spec.input_dtype} x/B, R={spec.R}, max_window={spec.W}"
                       + (f", Philox-{spec.philox_rounds} stochastic rounding" if spec.philox_rounds else ""),
           "ms_per_call": round(ms, 4), "algorithmic_bytes": nbytes,
           "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
           "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "us_per_request": round(ms * 1e3 / n, 3),
           "traffic_over_algorithmic": traffic_ratio(name)}
    ins = valu_instructions(name)
    if ins is not None:
        # the vector-ALU roofline: committed instruction count over this run's time
        out["valu_issue_frac"] = round(ins / VALU_PEAK_PER_S / (ms * 1e-3), 4)
    out.update(empty_launch_costs(dp, tabs, spec, stream))
    out["grid"] = rp.rssm_materialize_launch_config(
        num_layers=spec.L, batch=spec.B, num_heads=spec.H, heads_per_group=spec.hpg, dim=spec.dim,
        dstate=spec.dstate, max_window=spec.W, ring_buffer_len=spec.R, state_dtype=spec.state_dtype,
        input_dtype=spec.input_dtype, philox_rounds=spec.philox_rounds)[0]
    say(f"{name}: {out}")
    del call, tabs, dp
    torch.cuda.empty_cache()
    return out


def _counter_rows(path, counter):
    """(kernel name, value) per dispatch of one counter, in dispatch order."""
    import csv
    rows = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            d = int(r["Dispatch_Id"])
            name, v = rows.get(d, (r["Kernel_Name"], 0.0))
            rows[d] = (name, v + float(r["Counter_Value"]))
    return [rows[d] for d in sorted(rows)]


COUNTER_DESCRIPTION = {
    "large_bf16": "materialize_kernel<bf16 state, bf16 input, 64x128, kmax 8> on the large_bf16 workload "
                  "(48 layers, 256 active requests, 256 heads of 64x128 bf16)",
    "large_i8": "materialize_kernel<int8 state, fp16 input, 64x128, kmax 8> on the large_i8 workload "
                "(48 layers, 64 active requests, a quarter with k = 0, 256 heads of 64x128 int8 + fp32 row scales)",
    "large_f8sr": "materialize_kernel<e4m3 state, bf16 input, 64x128, kmax 16, Philox-10 stochastic rounding> on "
                  "the large_f8sr workload (48 layers, 128 active requests, 128 heads of 64x128 e4m3 + fp32 row scales)",
    "checkpoints": "materialize_kernel<bf16, bf16, 64x128, kmax 8, 4 checkpoints> on large_bf16 with two "
                   "checkpoints per request (in-place flush of all k tokens + the state after k//2 tokens)",
    "gdn_large": "gdn_commit_kernel<8> on gdn_large (48 layers, 256 requests, 32 value heads over 16 key heads, "
                 "fp32 128x128 states, 8-token bf16 windows, tracked steps)",
    "ssu_large": "ssu_decode_kernel<bf16, bf16, 4> on ssu_large (one layer, 256 requests, 256 heads of 64x128 bf16 "
                 "checkpoints, 4 new tokens)",
}


def counters_summary(fetch_csv, write_csv, alg_json):
    """HBM traffic of one kernel from FETCH_SIZE and WRITE_SIZE runs of
    `--pmc-calibrate` (KiB per dispatch).  The run ends with two 1 GiB device
    copies (1 GiB read and 1 GiB written each): their readings give the factor
    from counter KiB to bytes that is applied to the kernel's dispatches."""
    info = None
    for line in open(alg_json):
        line = line.strip()
        if line.startswith("{") and "counter_workload" in line:
            info = json.loads(line)
    if info is None:
        raise SystemExit(f"{alg_json}: no counter_workload line")
    wl, alg, kname = info["counter_workload"], int(info["algorithmic_bytes"]), info["kernel"]
    fetch = _counter_rows(fetch_csv, "FETCH_SIZE")
    write = _counter_rows(write_csv, "WRITE_SIZE")
    gib_kib = float(1 << 20)
    out = []
    facs = []
    for rows, what in ((fetch, "FETCH_SIZE"), (write, "WRITE_SIZE")):
        copies = [v for n, v in rows if "copyBuffer" in n][-2:]
        mats = [v for n, v in rows if kname in n]
        if len(copies) != 2 or not mats:
            raise SystemExit(f"{what}: expected 2 calibration copies and {kname} dispatches")
        facs.append((what, copies, mats, gib_kib / (sum(copies) / 2)))
    rd = sum(facs[0][2]) / len(facs[0][2]) * facs[0][3] * 1024
    wr = sum(facs[1][2]) / len(facs[1][2]) * facs[1][3] * 1024
    repo = "$REPO"
    out.append(f"# HBM traffic of {COUNTER_DESCRIPTION[wl]}; one call per dispatch")
    out.append("# commands (REPO = repository root on the MI355X machine):")
    for c, d in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        out.append(f"#   cd /tmp && rocprofv3 --pmc {c} --output-format csv -d /tmp/pmc_{d} -o {d} -- "
                   f"python3 {repo}/bench.py --pmc-calibrate --workload {wl} > /tmp/alg_{d}.json")
    out.append(f"#   python3 {repo}/bench.py --summarize-counters /tmp/pmc_fetch/fetch_counter_collection.csv "
               "/tmp/pmc_write/write_counter_collection.csv /tmp/alg_fetch.json")
    out.append("# calibration: the run ends with two torch copy_ of 1 GiB (__amd_rocclr_copyBuffer: 1 GiB read, "
               "1 GiB written)")
    for what, copies, mats, fac in facs:
        out.append(f"#   {what} per copy: {copies[0]:.1f}, {copies[1]:.1f} KiB -> factor {fac:.4f}")
    out.append(f"# {kname} dispatches: FETCH_SIZE " + ", ".join(f"{v:.1f}" for v in facs[0][2])
               + " KiB; WRITE_SIZE " + ", ".join(f"{v:.1f}" for v in facs[1][2]) + " KiB")
    out.append(f"counter_workload: {wl}")
    out.append(f"kernel_source_hash: {kernel_hash(COUNTER_SOURCES[wl])}")
    out.append(f"fetch_factor: {facs[0][3]:.4f}")
    out.append(f"write_factor: {facs[1][3]:.4f}")
    out.append(f"hbm_read_bytes_per_launch: {rd:.0f}")
    out.append(f"hbm_write_bytes_per_launch: {wr:.0f}")
    out.append(f"hbm_bytes_per_launch: {rd + wr:.0f}")
    out.append(f"algorithmic_bytes_per_launch: {alg}")
    out.append(f"traffic_over_algorithmic: {(rd + wr) / alg:.4f}")
    return "\n".join(out) + "\n"


def written_state_elements(spec, meta) -> int:
    """State elements one materialize call writes: every listed request's
    (layer) pairs whose source and destination are not the pad slot."""
    n = 0
    for b in meta.active:
        if b < 0 or b >= spec.B:
            break
        n += int(((meta.src[:, b] != spec.pad_slot_id) & (meta.dst[:, b] != spec.pad_slot_id)).sum())
    return n * spec.H * spec.dim * spec.dstate


VALU_HEADER = ("# workload | kernel | SQ_WAVES | SQ_INSTS_VALU | SQ_ACTIVE_INST_VALU | GRBM_GUI_ACTIVE | valu_time_ms | "
               "elements | VALU instr/element")


def valu_summary(counter_csv, bench_json):
    """One row of the vector-ALU table from a --pmc run of SQ_ACTIVE_INST_VALU,
    GRBM_GUI_ACTIVE, SQ_INSTS_VALU and SQ_WAVES over a profile-mode bench run,
    and the JSON line that run printed (its `valu_elements` is the per-element
    denominator).  Every dispatch of the workload reads alike; the last one is
    used.  valu_time_ms = SQ_INSTS_VALU * 4 cycles (a wave64 instruction on a
    16-lane SIMD) / 1024 SIMDs / 2.4 GHz, a lower bound on vector issue time
    (matrix-core instructions are counted as one instruction each)."""
    info = None
    for line in open(bench_json):
        line = line.strip()
        if line.startswith("{") and "valu_elements" in line:
            info = json.loads(line)
    if info is None:
        raise SystemExit(f"{bench_json}: no JSON line with valu_elements")
    lines = [ln for ln in pmc_summary(counter_csv).splitlines() if info["valu_kernel"] in ln]
    if not lines:
        raise SystemExit(f"{counter_csv}: no {info['valu_kernel']} dispatch")
    vals = dict(kv.split("=") for kv in lines[-1].split(": ", 1)[1].split())
    ins = float(vals["SQ_INSTS_VALU"])
    elems = int(info["valu_elements"])
    return (f"{info['valu_workload']} | {info['valu_kernel']} | {float(vals['SQ_WAVES']):.0f} | {ins:.4e} | "
            f"{float(vals['SQ_ACTIVE_INST_VALU']):.4e} | {float(vals['GRBM_GUI_ACTIVE']):.4e} | "
            f"{ins * 4 / 1024 / 2.4e9 * 1e3:.3f} | {elems} | {ins * 64 / elems:.2f}\n")


def pmc_summary(path):
    """One line per dispatch of a library kernel: dispatch id, kernel, then counter=value."""
    import csv
    rows = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if "rssm::" not in r["Kernel_Name"]:
                continue
            d = rows.setdefault(int(r["Dispatch_Id"]), {"": r["Kernel_Name"].split("(")[0].replace("void ", "")})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return "".join(f"dispatch {d} {c.pop('')}: " + " ".join(f"{k}={v:.6g}" for k, v in sorted(c.items())) + "\n"
                   for d, c in sorted(rows.items()))


def trace_summary(stats_csv):
    """Rows of rocprofv3's kernel_stats.csv: name | calls | average | min | max | total | percent (ns)."""
    import csv
    out = ["# rocprofv3 kernel stats (ns): name | calls | average | min | max | total | percent"]
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            out.append(f"{r['Name'][:110]} | {r['Calls']} | {float(r['AverageNs']):.0f} | {float(r['MinNs']):.0f} | "
                       f"{float(r['MaxNs']):.0f} | {float(r['TotalDurationNs']):.0f} | {float(r['Percentage']):.2f}")
    return "\n".join(out) + "\n"


if __name__ == "__main__":
    main()
