"""bench.py's single-GPU contract, checked without a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_cpu_baseline_leg_runs_single_and_threaded():
    """The oracle baseline leg on a small workload: single-threaded and one
    worker per core, both reported, the threaded figure as the value."""
    sys.path.insert(0, ROOT)
    import bench
    import synth
    sp = synth.spec(1, B=3)
    reqs = synth.request_draws(sp)
    inputs = {(0, r): synth.gen_layer_request(sp, 0, r, rq) for r, rq in enumerate(reqs)}
    res = bench.cpu_baseline(sp, inputs, len(reqs), 0.4)
    assert res["kind"] == "oracle" and res["unit"] == "layer-steps/s"
    assert res["value"] > 0 and res["single_thread"]["value"] > 0
    assert 1 <= res["cores"] <= 16
    assert res["single_thread"]["cores"] == 1


def test_bench_times_exactly_the_steps_asked_for():
    """The overlapped headline is timed over kvoff_step calls of up to one
    pass over the rotating layers; the calls add up to exactly --steps."""
    sys.path.insert(0, ROOT)
    import bench
    for n in range(0, 23):
        for per in (1, 3, 4):
            calls = bench.step_calls(n, per)
            assert sum(calls) == n
            assert all(1 <= c <= per for c in calls)
            assert calls[:-1] == [per] * (len(calls) - 1) if calls else True
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "0"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2 and "--steps" in r.stderr
