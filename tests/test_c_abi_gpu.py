"""The C ABI used from plain C (tests/c_abi/check.c, built by
__graft_entry__.build()): device memory from the HIP runtime, the entry
points of include/sda.h, results checked against the oracle inside the
program (see its header for the checks)."""
import json
import os
import subprocess

import pytest

from tests.gpu_util import say

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "check")


def test_c_program_against_oracle():
    assert os.path.exists(BIN), "tests/c_abi/check is not built: run __graft_entry__.build()"
    say("case: plain C consumer of libsda.so (3 instances, 24 rows, 700 cells)")
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    say(r.stdout.strip())
    if r.stderr.strip():
        say(r.stderr.strip())
    assert r.returncode == 0, f"exit {r.returncode}"
    line = [ln for ln in r.stdout.splitlines() if ln.startswith("{")][-1]
    d = json.loads(line)
    assert d["c_abi_check"] == "ok" and d["failures"] == 0
    assert d["rejected_status"]
