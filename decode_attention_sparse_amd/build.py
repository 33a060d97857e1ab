"""Build step for libsda.so (hipcc, gfx950) -- run on the host, no GPU needed.

    python -m decode_attention_sparse_amd.build

compiles every csrc/*.hip into decode_attention_sparse_amd/libsda.so.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libsda.so")
ARCH = "gfx950"

# packed fp32 instructions are disabled for the device code on purpose.
HIPCC_FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
               "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-munsafe-fp-atomics"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


PROBES = {
    # name: extra link flags.  gather_ceiling: the HBM read ceilings that
    # `bench.py --gather-ceiling` reports; valu_chunk: the vector-ALU chunk
    # pass variants timed beside the library (loads libsda.so at run time);
    # simd_placement: which SIMDs the waves of a workgroup land on.
    "gather_ceiling": [],
    "valu_chunk": ["-ldl"],
    "simd_placement": [],
}
PROBE_BIN = os.path.join(PKG, "probes", "gather_ceiling")


def build_probe(verbose: bool = False) -> str:
    """The standalone measurement programs under probes/ (not part of the library)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    for name, link in PROBES.items():
        src = os.path.join(PKG, "probes", name + ".hip")
        out = os.path.join(PKG, "probes", name)
        tmp = out + ".tmp%d" % os.getpid()
        cmd = [hipcc, "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-Xclang", "-target-feature",
               "-Xclang", "-packed-fp32-ops", src, "-o", tmp, *link]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stderr}")
        os.replace(tmp, out)
    return PROBE_BIN


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, *HIPCC_FLAGS, *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that is harmless
    noise = "not a recognized feature for this target"
    err = "\n".join(ln for ln in r.stderr.splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_probe(verbose=True))
