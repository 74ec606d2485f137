"""Host-side checks of the gfx950 code the GEMM compiles to (no GPU needed).

The bf16 GEMM stages its operands with LDS DMA issued from inline assembly:
each copy sets M0 to the LDS address and then issues
global_load_lds_dwordx4. That is only sound while nothing else in the kernel
relies on M0, so every use of M0 in the compiled code must belong to such a
copy.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "target_aware_latent_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _device_asm(src):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    cmd = [HIPCC, "--offload-arch=gfx950", "--cuda-device-only", "-S", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-o", "-", os.path.join(CSRC, src)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return res.stdout


def test_m0_written_only_by_lds_dma():
    asm = _device_asm("gemm.hip")
    lines = [l.strip() for l in asm.splitlines()]
    code = [l for l in lines if l and not l.startswith((";", ".", "//")) and not l.endswith(":")]
    dma = 0
    for i, l in enumerate(code):
        if re.search(r"\bm0\b", l):
            # the only accepted use: s_mov_b32 m0, sN ; s_nop 0 ; global_load_lds_dwordx4
            assert re.fullmatch(r"s_mov_b32 m0, s\d+", l), f"unexpected use of m0: {l}"
            assert code[i + 1] == "s_nop 0", code[i + 1]
            assert code[i + 2].startswith("global_load_lds_dwordx4"), code[i + 2]
            dma += 1
    assert dma > 0, "no LDS DMA copies found in the GEMM"

