"""Checks on the gfx950 assembly of the library's kernels (CPU only: the
sources are compiled to assembly here). Every kernel runs without scratch
memory (no register spills), and in the GEMM kernels the only use of M0 is
the write that sets the LDS base of a direct global-to-LDS load, which the
inline assembly clobbers."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp8_scaled_gemm_amax_amd", "csrc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off", "-Xclang", "-target-feature",
         "-Xclang", "-packed-fp32-ops", "--cuda-device-only", "-S", "-o", "-"]


@pytest.fixture(scope="module", params=["gemm.hip", "quant.hip", "moe.hip"])
def asm(request):
    out = subprocess.run(["/opt/rocm/bin/hipcc", *FLAGS, os.path.join(CSRC, request.param)], capture_output=True,
                         text=True)
    if out.returncode != 0:
        pytest.fail(out.stderr[-2000:])
    return request.param, out.stdout


def kernels(text):
    """name -> body of every kernel function in the assembly (to its end label,
    so code after an early s_endpgm is included)."""
    res = {}
    for m in re.finditer(r"^(_Z\w+):[^\n]*$(.*?)^\.Lfunc_end\d+:", text, flags=re.M | re.S):
        res[m.group(1)] = m.group(2)
    return res


def test_no_scratch(asm):
    name, text = asm
    sizes = re.findall(r"\.private_segment_fixed_size:\s*(\d+)", text)
    assert sizes and all(int(s) == 0 for s in sizes), f"{name}: a kernel uses scratch memory"
    assert "scratch_" not in text


def test_m0_only_feeds_direct_loads(asm):
    name, text = asm
    found = kernels(text)
    assert len(found) == len(re.findall(r"^\.Lfunc_end\d+:", text, flags=re.M)) > 0, "kernel bodies not found"
    for kname, body in found.items():
        lines = [l.strip() for l in body.splitlines() if l.strip() and not l.strip().startswith(";")]
        for i, l in enumerate(lines):
            if re.search(r"\bm0\b", l):
                # (from any scalar register: vcc_lo is one the allocator also hands out)
                assert re.match(r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)$", l), (kname, l)
                # one wait state before a load with a VGPR address; five before one
                # whose SGPR base came from v_readfirstlane
                assert lines[i + 1] in ("s_nop 0", "s_nop 4") and \
                    re.match(r"global_load_lds_dword(x4)? ", lines[i + 2]), (kname, l)
