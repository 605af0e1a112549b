"""bench.py's contract: on the host, more than one GPU is refused with a message (the library
has no multi-GPU path; the bench measures one GPU), the help text lists the workload options and
the CPU baseline legs report per stage; on the GPU, a short run prints the JSON line."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_help_lists_the_options():
    r = _run("--help")
    assert r.returncode == 0
    for opt in ("--steps", "--warmup", "--workload", "--alignment", "--route-groups", "--fp8", "--backward", "--graph",
                "--no-graph", "--bf16-partials", "--seed"):
        assert opt in r.stdout


def test_help_lists_the_flush_option():
    out = _run("--help").stdout
    assert "--no-flush" in out and "--stream-ceiling" in out


def test_cpu_baseline_legs_on_the_host():
    """The CPU-baseline leg on workload 1 (the small float32 workload), forward, FP8-free and
    backward: both legs report a rate, the all-cores leg names its threads and the host."""
    sys.path.insert(0, ROOT)
    import bench
    import workloads as wl

    c = wl.WORKLOADS[1]
    key = wl.workload_key(1)
    logits = wl.router_logits(key, c["T"], c["E"], zipf_s=c["zipf_s"])
    x = wl.hidden_states(key, c["T"], c["H"], c["dtype"])
    for backward in (False, True):
        r = bench.cpu_baseline(c, key, logits, x, None, 0, 0, 0, 10 ** 7, backward=backward)
        assert r["kind"] == "oracle" and r["value"] > 0 and r["single_thread"]["value"] > 0
        assert 1 <= r["cores"] <= 16 and r["host"]["threads_used"] == r["cores"]
        assert r["host"]["nproc"] >= 1 and r["host"]["usable_cores"] >= 1 and r["host"]["cpu_model"]
        stages = ("combine_bwd", "dispatch_bwd", "route_bwd") if backward else ("route", "index", "dispatch", "combine")
        for leg in (r, r["single_thread"]):
            st = leg["stage_seconds_median"]
            assert tuple(st) == stages and all(v >= 0 for v in st.values())
            assert sum(st.values()) <= 2 * leg["seconds_per_pass"] + 0.05


def test_cpu_baseline_fp8_and_group_modes():
    sys.path.insert(0, ROOT)
    import bench
    import workloads as wl

    c = dict(wl.WORKLOADS[4], T=256, H=256)  # workload 4's layout at a host-friendly size
    key = (4000,)
    logits = wl.router_logits(key, c["T"], c["E"], zipf_s=c["zipf_s"])
    x = wl.hidden_states(key, c["T"], c["H"], c["dtype"])
    y = wl.expert_outputs(key, c["T"] * c["K"], c["H"], c["dtype"])
    for fp8, bf16p, rg in ((True, False, 0), (False, True, 4), (True, True, 4)):
        r = bench.cpu_baseline(c, key, logits, x, y, 0, 0, rg, 10 ** 7, bf16_partials=bf16p, fp8=fp8)
        assert r["value"] > 0 and ("FP8" in r["sample"]) == fp8


def test_pmc_summary_names_follow_workload_and_mode():
    """The roofline's traffic is read from the PMC summary of the same workload and mode: an
    aligned or group-limited run does not pick up the plain workload's counters."""
    sys.path.insert(0, ROOT)
    import bench

    assert bench.profile_tag(3) == "workload3"
    assert bench.profile_tag(3, alignment=128) == "workload3_align128"
    assert bench.profile_tag(4, route_groups=4) == "workload4_groups4"
    assert bench.profile_tag(4, backward=True) == "workload4_bwd"
    assert bench.profile_tag(4, fp8=True) == "workload4_fp8"
    assert bench.profile_tag(4, bf16_partials=True) == "workload4_bf16p"
    names = set(os.listdir(os.path.join(ROOT, "profiles")))
    for f in names:
        if f.endswith("__pmc.txt"):
            tag = f.split("__")[1]
            assert tag.startswith("workload"), f


@pytest.mark.gpu
def test_bench_line_on_the_gpu():
    """A short bench run (workload 1, forward and backward) prints one JSON line with the fields
    the bench contract names, both launch modes timed and a roofline on a named call."""
    import json
    for extra in ((), ("--backward",)):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "1", "--steps", "3",
                            "--warmup", "1", "--no-cpu-baseline", *extra], capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stderr[-2000:]
        lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
        assert len(lines) == 1
        d = json.loads(lines[0])
        for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                  "vs_baseline", "dtype", "data", "config", "roofline"):
            assert k in d, k
        assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["value"] > 0
        assert d["config"]["workload"] and d["launch"] == "eager"
        assert set(d["ms_per_step_by_launch"]) == {"eager", "hip graph replay"}
        rf = d["roofline"]
        assert rf["bound"] == "hbm" and rf["peak"] == 8000.0 and 0 < rf["frac"] < 1 and rf["call"] in d["kernel_us"]
