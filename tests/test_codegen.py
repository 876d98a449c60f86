"""Code-generation guards for the HIP kernels (CPU only: hipcc cross-compiles gfx950).

A kernel whose helper lambdas get outlined into real device functions passes its
accumulators through private (scratch) memory: still correct, but an order of
magnitude slower.  These tests compile each kernel source to gfx950 assembly and
require that no kernel calls a function or touches scratch memory.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "convolution_int8_implicit_amd", "csrc")
HIPCC = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)


@pytest.mark.skipif(HIPCC is None, reason="hipcc not available")
@pytest.mark.parametrize("src", ["igemm.hip", "conv1x1.hip", "stem.hip"])
def test_kernels_stay_in_registers(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    assert "s_swappc_b64" not in asm, f"{src}: a kernel calls an outlined device function"
    assert not re.search(r"^\s+scratch_(load|store)", asm, re.M), f"{src}: a kernel uses scratch memory"
    sizes = [int(v) for v in re.findall(r"\.private_segment_fixed_size:\s+(\d+)", asm)]
    assert sizes and max(sizes) == 0, f"{src}: private segment sizes {sizes}"
