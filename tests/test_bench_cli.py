"""bench.py's command line on the CPU: more than one GPU is refused with a message and exit status 2
before any GPU work (the path has no multi-GPU leg), and the help lists the measurements."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    p = _run("--gpus", "2")
    assert p.returncode == 2
    assert "one GPU only" in p.stderr
    assert p.stdout == ""


def test_help_lists_the_measurements():
    p = _run("--help")
    assert p.returncode == 0
    for word in ("--config", "--measure", "--separate", "--grouped", "--partition"):
        assert word in p.stdout


def test_cpu_baseline_legs_on_the_tiny_workload():
    """The oracle's two timing legs (one worker process per host core, and one thread) run on a
    small workload and report their core counts and rates."""
    sys.path.insert(0, ROOT)
    import bench
    from workloads import config
    allcore, one = bench.cpu_baselines(config(1), 0.2)
    assert 1 <= allcore["cores"] <= 16 and one["cores"] == 1
    for r in (allcore, one):
        assert r["kind"] == "oracle" and r["unit"] == "GB/s"
        assert r["value"] > 0 and r["attended_tokens_per_s"] > 0
