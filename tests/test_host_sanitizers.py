"""The host code under the CPU sanitizers (no GPU needed).

- The oracle and the seeded generator (plain C), every function on small
  inputs and their edge cases: address and undefined-behaviour sanitizers.
- The library's host-only code, the admission policy and the status strings,
  over its whole input space: address and undefined-behaviour sanitizers.
- The staged recall engine's worker pool, driven as the engine drives it:
  the thread sanitizer, and separately the address and undefined-behaviour
  sanitizers.

Each program is built with gcc/g++ from the committed sources and must print
PASS with no sanitizer report (reports abort the program: exit status not 0).
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
C = os.path.join(ROOT, "tests", "c")
CSRC = os.path.join(ROOT, "sparse_kv_cache_mean_amd", "csrc")
ASAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
           TSAN_OPTIONS="halt_on_error=1:second_deadlock_stack=1")


def _build_and_run(tmp_path, name, compiler, flags, srcs, incs, libs=()):
    exe = os.path.join(str(tmp_path), name)
    cmd = [compiler, "-O1", "-g", *flags, *[f"-I{i}" for i in incs], *srcs, "-o", exe, *libs]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, f"build failed: {' '.join(cmd)}\n{b.stderr}"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=ENV)
    assert r.returncode == 0, f"{name} exited {r.returncode}:\n{r.stderr[-4000:]}"
    assert r.stdout.strip().startswith("PASS"), r.stdout
    return r.stdout.strip()


def test_oracle_and_generator_under_address_and_ub_sanitizers(tmp_path):
    _build_and_run(tmp_path, "oracle_sanitize", "gcc", ["-std=c11", "-fopenmp", *ASAN],
                   [os.path.join(C, "oracle_sanitize.c"), os.path.join(ROOT, "oracle", "kvoff_oracle.c"),
                    os.path.join(ROOT, "synth", "synth.c")],
                   [os.path.join(ROOT, "oracle"), os.path.join(ROOT, "synth")], ["-lm"])


def test_admission_policy_under_address_and_ub_sanitizers(tmp_path):
    out = _build_and_run(tmp_path, "host_policy", "g++", ["-std=c++17", *ASAN],
                         [os.path.join(C, "host_policy_test.cpp"),
                          os.path.join(CSRC, "admission_policy.cpp"),
                          os.path.join(CSRC, "host_errors.cpp")],
                         [os.path.join(ROOT, "include"), CSRC])
    assert int(out.split()[1]) > 10000


@pytest.mark.parametrize("flags", [["-fsanitize=thread"], ASAN], ids=["thread", "address-ub"])
def test_staged_worker_pool_under_sanitizers(tmp_path, flags):
    _build_and_run(tmp_path, "stage_pool", "g++", ["-std=c++17", "-pthread", *flags],
                   [os.path.join(C, "stage_pool_test.cpp")], [CSRC])
