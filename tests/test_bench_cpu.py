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
