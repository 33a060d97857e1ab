"""The prompt kernel issues its LDS-DMA loads from inline assembly that sets
M0, a register the compiler reserves for itself; that is sound only while no
other instruction of that kernel reads or writes M0.  This compiles
chunk_mfma.hip for gfx950 (host only, no GPU) and checks, in
prompt_dma_kernel's code, that every M0 reference is an `s_mov_b32 m0, sN`
immediately followed by the global_load_lds_dwordx4 that uses it, and that
the kernel has no other LDS-DMA load and no register spills."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_sparse_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which("hipcc")), reason="no hipcc")
def test_prompt_dma_kernel_m0_use(tmp_path):
    out = tmp_path / "chunk_mfma.s"
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "--cuda-device-only", "-S", "-o", str(out), "-I", CSRC,
           os.path.join(CSRC, "chunk_mfma.hip")]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    m = re.search(r"^(_ZN\S*prompt_dma_kernel\S*):", asm, re.M)
    assert m, "prompt_dma_kernel not found"
    body = asm[m.end():asm.index("s_endpgm", m.end())]
    lines = [ln.split(";")[0].strip() for ln in body.splitlines()]
    lines = [ln for ln in lines if ln and not ln.startswith(".")]
    n_dma = 0
    for k, ln in enumerate(lines):
        if re.search(r"\bm0\b", ln):
            assert re.fullmatch(r"s_mov_b32 m0, s\d+", ln), f"other use of m0: {ln}"
            assert k + 1 < len(lines) and lines[k + 1].startswith("global_load_lds_dwordx4"), \
                f"m0 set without its load: {ln} / {lines[k + 1] if k + 1 < len(lines) else ''}"
        if "_lds_" in ln and ln.startswith(("global_load", "buffer_load")):
            n_dma += 1
            assert re.search(r"\bm0\b", lines[k - 1]), f"LDS-DMA load without its m0: {ln}"
    assert n_dma > 0
    i = asm.index(".name:           " + m.group(1))
    j = asm.find(".agpr_count", i)
    meta = asm[i:j if j > 0 else len(asm)]  # this kernel's metadata fields after its name
    assert re.search(r"\.vgpr_spill_count:\s+0\b", meta), meta[:400]
