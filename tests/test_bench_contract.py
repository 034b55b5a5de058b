"""CPU checks of the benchmark's command-line contract (no GPU work is started)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_workloads_are_listed():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0
    for w in ("step480", "step720", "rollout480", "rollout65s", "plan480", "bc480", "bc720"):
        assert w in r.stdout


def test_cpu_baseline_parts_run_on_the_host():
    """The CPU-baseline record's host description and its 1-thread tiny rollout."""
    sys.path.insert(0, ROOT)
    import bench
    info = bench._host_info()
    assert info["cpu_model"] and info["blas"] and info["affinity_cores"] >= 1
    tiny = bench.tiny_rollout_one_thread()
    assert tiny["calls"] == 108 and tiny["seconds"] > 0 and tiny["gflops"] > 0


def test_step_statistics_and_clock_sampler():
    sys.path.insert(0, ROOT)
    import bench

    class Ev:
        def __init__(self, t):
            self.t = t

        def elapsed_time(self, other):
            return other.t - self.t

    st = bench.step_stats([(Ev(0.0), Ev(x)) for x in (3.0, 1.0, 2.0, 5.0)])
    assert st == {"median": 3.0, "min": 1.0, "mean": 2.75, "n": 4}
    out = bench.ClockSampler().start().stop()
    assert set(out) == {"sclk_mhz", "mclk_mhz", "source"}
