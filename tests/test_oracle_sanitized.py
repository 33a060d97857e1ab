"""The fp64 oracle under AddressSanitizer and UndefinedBehaviorSanitizer: a C
driver (tests/sanitize/oracle_check.c) calls every oracle function on small
inputs with masked pages, out-of-range ids and edge counts, and checks that
the merge of the chunk partials equals the direct attention.  Host only."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    exe = str(tmp_path / "oracle_check")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(HERE, "sanitize", "oracle_check.c"), os.path.join(ROOT, "oracle", "oracle.c"),
           "-lm", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and ("asan" in r.stderr or "ubsan" in r.stderr):
        pytest.skip("sanitizer runtimes not available: " + r.stderr.strip()[-200:])
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.strip() == "ok", run.stdout + run.stderr
    assert "runtime error" not in run.stderr, run.stderr
