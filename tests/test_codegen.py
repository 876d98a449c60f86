"""Code-generation guards for the HIP kernels (CPU only: hipcc cross-compiles gfx950).

Each kernel source is compiled to gfx950 assembly once (in parallel) and checked for:
  * no function calls or scratch memory: a kernel whose helper lambdas get outlined into real
    device functions passes its accumulators through private (scratch) memory, still correct
    but an order of magnitude slower;
  * persistent grids that fit: workgroups assumed resident together fit the registers and LDS;
  * DPP moves (the stem's pooling) outside exec-masked regions;
  * no workgroup barrier reached with LDS reads outstanding: the kernels refill LDS (buffer->LDS
    DMA or ds_write) right after a barrier, assuming every wave's reads of it are complete, but
    s_barrier does not wait for a wave's LDS reads and the compiler may sink a step's last
    fragment reads past the next barrier.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "convolution_int8_implicit_amd", "csrc")
HIPCC = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)
SOURCES = ["igemm.hip", "conv1x1.hip", "stem.hip"]


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    """{source: gfx950 assembly text}, the sources compiled in parallel."""
    if HIPCC is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm")

    def compile_one(src):
        dst = out / (src + ".s")
        cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               os.path.join(CSRC, src), "-o", str(dst)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return src, dst.read_text()

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        return dict(ex.map(compile_one, SOURCES))


@pytest.mark.parametrize("src", SOURCES)
def test_kernels_stay_in_registers(assembly, src):
    asm = assembly[src]
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


@pytest.mark.parametrize("src,kernel,per_cu_name", [
    ("stem.hip", "stem_kernel", "kStemPerCu"),
    # the chained and ring kernels size their grids as two workgroups per CU for four waves, one
    # for eight (their layout structs' PER_CU)
    ("conv1x1.hip", "conv1x1_chain_kernel", None),
    ("conv1x1.hip", "conv1x1_ring_kernel", None),
    # the haloed-window kernels: two four-wave workgroups per CU (the 3x3 over 128+ channels),
    # one of eight waves (the 64-channel one)
    ("igemm.hip", "conv3x3_win_kernel", None),
    ("igemm.hip", "conv3x3_halo_kernel", None),
])
def test_persistent_residency_fits(assembly, src, kernel, per_cu_name):
    """A grid sized as per_cu workgroups per CU assumes they are all resident: their waves must
    fit the 512 registers of a SIMD lane and their LDS the CU's 160 KB."""
    per_cu = None
    if per_cu_name:
        text = open(os.path.join(CSRC, src)).read()
        per_cu = int(re.search(rf"constexpr int {per_cu_name} = (\d+);", text).group(1))
    res = {k: v for k, v in _kernel_resources(assembly[src]).items() if kernel in k}
    assert res, f"no {kernel} found"
    for name, f in res.items():
        pc = per_cu if per_cu is not None else {256: 2, 512: 1}[f["max_flat_workgroup_size"]]
        waves_per_simd = pc * f["max_flat_workgroup_size"] // 64 // 4
        regs = f["vgpr_count"] + f.get("agpr_count", 0)
        assert waves_per_simd * regs <= 512, (name, f)
        assert pc * f["group_segment_fixed_size"] <= 160 * 1024, (name, f)


def test_stem_dpp_moves_run_in_every_lane(assembly):
    """The stem pools across lanes with DPP moves.  A DPP read of a lane that the exec mask has
    switched off returns the old value, so no DPP move may sit inside an exec-masked region."""
    total = 0
    for body in re.split(r"\n(?=_Z\S*stem_kernel\S*:)", assembly["stem.hip"])[1:]:
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


def barriers_with_pending_reads(asm: str):
    """(kernel, line) for each s_barrier reached with LDS reads outstanding, counting ds_reads and
    the s_waitcnt lgkmcnt instructions in straight-line order."""
    out = []
    for name in re.findall(r"^(_Z\w*kernel\w*):", asm, re.M):
        body = asm[asm.index(name + ":"):]
        body = body[:body.index(".Lfunc_end")]
        pending = 0
        for n, line in enumerate(body.split("\n")):
            t = line.strip()
            if t.startswith("ds_read"):
                pending += 1
            elif t.startswith("s_waitcnt") and "lgkmcnt" in t:
                pending = min(pending, int(re.search(r"lgkmcnt\((\d+)\)", t).group(1)))
            elif t.startswith("s_barrier") and pending:
                out.append((name, n))
    return out


def test_barrier_scan_on_a_planted_case():
    """The scan itself: a barrier after an unwaited read is reported, a waited one is not."""
    asm = ("_Zk1_kernel:\n ds_read_b128 v[0:3], v4\n s_barrier\n s_waitcnt lgkmcnt(0)\n.Lfunc_end0:\n"
           "_Zk2_kernel:\n ds_read_b128 v[0:3], v4\n s_waitcnt lgkmcnt(0)\n s_barrier\n.Lfunc_end1:\n")
    assert barriers_with_pending_reads(asm) == [("_Zk1_kernel", 2)]


@pytest.mark.parametrize("src", SOURCES)
def test_no_barrier_with_lds_reads_in_flight(assembly, src):
    bad = barriers_with_pending_reads(assembly[src])
    assert not bad, bad[:10]
