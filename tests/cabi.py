"""Builds tests/c/abi_roundtrip.c: a C program that drives libkvoff.so through
include/kvoff.h alone and checks it against the C oracle (test infrastructure)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c", "abi_roundtrip.c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(out_dir: str) -> str:
    exe = os.path.join(out_dir, "abi_roundtrip")
    lib_dir = os.path.join(ROOT, "sparse_kv_cache_mean_amd")
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "oracle"),
           "-I", os.path.join(ROOT, "synth"), "-I", os.path.join(ROCM, "include"),
           SRC, os.path.join(ROOT, "oracle", "kvoff_oracle.c"),
           os.path.join(ROOT, "synth", "synth.c"), "-o", exe,
           "-L", lib_dir, "-lkvoff", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-fopenmp", "-lm", f"-Wl,-rpath,{lib_dir}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
    return exe
