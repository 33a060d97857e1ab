"""The C ABI's host logic under AddressSanitizer and UndefinedBehaviorSanitizer:
the library is rebuilt with host-side sanitizers (device code as usual), and
a C driver (tests/sanitize/abi_check.c) calls every entry point with
arguments it must reject before any device work and sweeps the geometry
helpers over their edges.  Host only: nothing launches."""
import glob
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "decode_attention_sparse_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]


def test_abi_host_logic_under_sanitizers(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("no ROCm compilers")
    objs, procs = [], []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = str(tmp_path / (os.path.basename(src)[:-4] + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen(
            [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN,
             "-fno-omit-frame-pointer", "-I", CSRC, "-c", src, "-o", obj],
            stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    for pr in procs:
        _, err = pr.communicate(timeout=600)
        assert pr.returncode == 0, err
    lib = str(tmp_path / "libsda_san.so")
    r = subprocess.run([HIPCC, "-shared", "-fPIC", *SAN, *objs, "-o", lib],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    exe = str(tmp_path / "abi_check")
    r = subprocess.run([CLANG, "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
                        "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
                        os.path.join(HERE, "sanitize", "abi_check.c"), "-L", str(tmp_path),
                        "-lsda_san", "-Wl,-rpath," + str(tmp_path), "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.strip() == "ok", run.stdout + run.stderr
    assert "runtime error" not in run.stderr, run.stderr
    assert "AddressSanitizer" not in run.stderr, run.stderr
