"""bench.py keeps its output contract in every mode: one JSON line with the
metric, the whole-job value, the roofline object and the CPU-baseline field.

The GPU cases run bench.py as a child process with few steps (timing values
are not checked, only that each mode runs and reports)."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def run_bench(*args, env=None, timeout=300):
    return subprocess.run([sys.executable, BENCH, *args], cwd=ROOT, env=env,
                          stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True,
                          timeout=timeout)


@pytest.mark.parametrize("how", ["flag", "env"])
def test_more_than_one_gpu_is_refused(how):
    env = dict(os.environ)
    args = []
    if how == "flag":
        args = ["--gpus", "2"]
    else:
        env["WORLD_SIZE"] = "2"
    res = run_bench(*args, env=env, timeout=60)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


CONTRACT_KEYS = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                 "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                 "roofline", "cpu_baseline")

MODES = {
    "headline": ["--no-cpu-baseline"],
    "tiny_f32_with_cpu_baseline": ["--workload", "tiny_f32"],
    "rope": ["--rope", "--no-cpu-baseline"],
    "bwd": ["--bwd"],
    "decode": ["--workload", "decode_b64_kv8192", "--no-cpu-baseline"],
    "decode_graph": ["--workload", "decode_b8_kv4097", "--graph", "--no-cpu-baseline"],
}


@pytest.mark.gpu
@pytest.mark.parametrize("mode", sorted(MODES))
def test_bench_modes_report_the_contract(mode):
    steps = "10" if "--graph" in MODES[mode] else "2"
    print(f"bench.py mode {mode}", flush=True)
    res = run_bench(*MODES[mode], "--steps", steps, "--warmup", "1")
    assert res.returncode == 0, res.stderr[-2000:]
    line = res.stdout.strip().splitlines()[-1]
    out = json.loads(line)
    for key in CONTRACT_KEYS:
        assert key in out, key
    assert out["n_gpus"] == 1 and out["steps"] == int(steps) and out["warmup"] == 1
    assert out["value"] > 0 and out["ms_per_step"] > 0
    assert isinstance(out["config"].get("workload"), str)
    roof = out["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] in ("hbm", "mfma", "alu")
    assert 0 < roof["frac"] < 1
    launch = out["config"].get("ms_per_launch")
    if "--graph" in MODES[mode]:
        assert launch is None
    else:
        assert launch["n"] == int(steps)
        assert 0 < launch["min"] <= launch["median"] <= launch["max"]
    if mode == "tiny_f32_with_cpu_baseline":
        cb = out["cpu_baseline"]
        assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
        assert cb["sample"]
    else:
        assert out["cpu_baseline"] is None


@pytest.mark.gpu
def test_copy_calibration_runs():
    res = run_bench("--copy-bytes", str(1 << 20), "--steps", "2", "--warmup", "1")
    assert res.returncode == 0, res.stderr[-2000:]
    out = json.loads(res.stdout.strip().splitlines()[-1])
    assert out["copy_bytes"] == 1 << 20 and out["ms_per_copy"] > 0


def test_kernel_digest_does_not_depend_on_the_tree_location():
    """The profiles' kernel digest hashes the sources and the compiler
    flags, but no path: the same build gets the same digest wherever the
    tree is checked out (CPU only)."""
    sys.path.insert(0, ROOT)
    import bench
    flags = bench._build_flags().decode()
    assert ROOT not in flags
    assert not any(os.path.isabs(f) for f in flags.split())
