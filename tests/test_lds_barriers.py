"""The kernels refill LDS (buffer->LDS DMA or ds_write) right after a workgroup barrier, on the
assumption that every wave's reads of that memory are complete when the barrier opens.  s_barrier
itself does not wait for a wave's outstanding LDS reads, and the compiler may sink a step's last
fragment reads (with their s_waitcnt) past the next barrier.  This check compiles the device code
to gfx950 assembly and requires that no s_barrier is reached with a ds_read still outstanding, as
counted from the s_waitcnt lgkmcnt instructions in straight-line order."""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "convolution_int8_implicit_amd", "csrc")
HIPCC = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)


def barriers_with_pending_reads(asm: str):
    """(kernel, barrier line) for each s_barrier reached with LDS reads outstanding."""
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


def test_counter_on_a_planted_case():
    """The scan itself: a barrier after an unwaited read is reported, a waited one is not."""
    asm = ("_Zk1_kernel:\n ds_read_b128 v[0:3], v4\n s_barrier\n s_waitcnt lgkmcnt(0)\n.Lfunc_end0:\n"
           "_Zk2_kernel:\n ds_read_b128 v[0:3], v4\n s_waitcnt lgkmcnt(0)\n s_barrier\n.Lfunc_end1:\n")
    assert barriers_with_pending_reads(asm) == [("_Zk1_kernel", 2)]


SOURCES = ["igemm.hip", "conv1x1.hip", "stem.hip"]


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    """The three kernel sources compiled to gfx950 assembly, in parallel."""
    if HIPCC is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm")

    def compile_one(src):
        dst = out / (src + ".s")
        cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-I", os.path.join(ROOT, "include"), "-I",
               CSRC, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "--cuda-device-only", "-S",
               os.path.join(CSRC, src), "-o", str(dst)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        return src, r.returncode, r.stderr[-2000:], dst

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        return {src: (rc, err, dst) for src, rc, err, dst in ex.map(compile_one, SOURCES)}


@pytest.mark.parametrize("src", SOURCES)
def test_no_barrier_with_lds_reads_in_flight(assembly, src):
    rc, err, dst = assembly[src]
    assert rc == 0, err
    bad = barriers_with_pending_reads(dst.read_text())
    assert not bad, bad[:10]
