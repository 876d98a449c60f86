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


def _kernel_resources(asm: str):
    """{kernel symbol: {field: int}} from the code object metadata of a gfx950 assembly file."""
    out = {}
    for block in asm.split("  - .agpr_count:")[1:]:
        block = ".agpr_count:" + block
        name = re.search(r"\.name:\s+(\S+)", block)
        if not name:
            continue
        fields = {}
        for key in ("agpr_count", "vgpr_count", "group_segment_fixed_size", "max_flat_workgroup_size"):
            m = re.search(rf"\.{key}:\s+(\d+)", block)
            if m:
                fields[key] = int(m.group(1))
        out[name.group(1)] = fields
    return out


@pytest.mark.skipif(HIPCC is None, reason="hipcc not available")
@pytest.mark.parametrize("src,kernel,per_cu_name", [
    ("stem.hip", "stem_kernel", "kStemPerCu"),
    # the chained and ring kernels size their grids as two workgroups per CU for four waves, one
    # for eight (their layout structs' PER_CU)
    ("conv1x1.hip", "conv1x1_chain_kernel", None),
    ("conv1x1.hip", "conv1x1_ring_kernel", None),
])
def test_persistent_residency_fits(src, kernel, per_cu_name, tmp_path):
    """A persistent grid sized as per_cu workgroups per CU assumes they are all resident: their
    waves must fit the 512 registers of a SIMD lane and their LDS the CU's 160 KB."""
    path = os.path.join(CSRC, src)
    per_cu = None
    if per_cu_name:
        per_cu = int(re.search(rf"constexpr int {per_cu_name} = (\d+);", open(path).read()).group(1))
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", path, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    res = {k: v for k, v in _kernel_resources(out.read_text()).items() if kernel in k}
    assert res, f"no {kernel} found"
    for name, f in res.items():
        pc = per_cu if per_cu is not None else {256: 2, 512: 1}[f["max_flat_workgroup_size"]]
        waves_per_simd = pc * f["max_flat_workgroup_size"] // 64 // 4
        regs = f["vgpr_count"] + f.get("agpr_count", 0)
        assert waves_per_simd * regs <= 512, (name, f)
        assert pc * f["group_segment_fixed_size"] <= 160 * 1024, (name, f)


@pytest.mark.skipif(HIPCC is None, reason="hipcc not available")
def test_stem_dpp_moves_run_in_every_lane(tmp_path):
    """The stem pools across lanes with DPP moves.  A DPP read of a lane that the exec mask has
    switched off returns the old value, so no DPP move may sit inside an exec-masked region."""
    out = tmp_path / "stem.s"
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", os.path.join(CSRC, "stem.hip"),
           "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    total = 0
    for body in re.split(r"\n(?=_Z\S*stem_kernel\S*:)", out.read_text())[1:]:
        body = body.split("s_endpgm")[0]
        depth = 0
        for line in body.split("\n"):
            if "s_and_saveexec" in line:
                depth += 1
            elif re.search(r"s_or_b64\s+exec", line):
                depth = max(0, depth - 1)
            elif "_dpp" in line:
                total += 1
                assert depth == 0, f"DPP move under a partial exec mask: {line.strip()}"
    assert total > 0
