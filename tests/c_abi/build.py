"""Build tests/c_abi/check (a plain C consumer of libsda.so, checked against
the oracle) with gcc: no HIP code in it, only the HIP runtime's C API.
Called by __graft_entry__.build(); needs libsda.so and oracle/liboracle.so."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "check.c")
BIN = os.path.join(HERE, "check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    pkg = os.path.join(ROOT, "decode_attention_sparse_amd")
    orc = os.path.join(ROOT, "oracle")
    tmp = BIN + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
           "-o", tmp, "-L", pkg, "-lsda", "-L", orc, "-loracle", "-L", os.path.join(ROCM, "lib"),
           "-lamdhip64", "-lm",
           # found next to the binary wherever the tree is copied
           "-Wl,-rpath,$ORIGIN/../../decode_attention_sparse_amd:$ORIGIN/../../oracle:"
           + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed ({r.returncode}):\n{r.stderr}")
    os.replace(tmp, BIN)
    return BIN


if __name__ == "__main__":
    print(build())
