"""The whole path driven from C through include/kvoff.h (no Python between
the caller and the library), checked against the C oracle inside the
program: digests, selection, recalled bytes, transfer count, attention."""
import subprocess

import pytest

from tests import cabi

pytestmark = pytest.mark.gpu


def test_c_program_round_trip(tmp_path):
    exe = cabi.build(str(tmp_path))
    print("[c abi] running", exe, flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip().endswith("PASS")
