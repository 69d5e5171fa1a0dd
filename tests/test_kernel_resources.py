"""Compiler resource checks of the GEMM kernels (no GPU needed).

The pipelined k loops wait for their global->LDS loads with counted waits
(`s_waitcnt vmcnt(N)`: "at most N load instructions still outstanding"), which
is only right when nothing else touches vector memory inside the loop.  A
VGPR spill would put scratch loads and stores there, so every GEMM kernel must
compile without VGPR spills and without scratch memory (SGPRs the compiler
parks in VGPR lanes touch no memory and are allowed).  The check compiles the sources
for gfx950 with the build's own flags and reads the compiler's resource
remarks.

"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "grouped_gemm_router_amd", "csrc")
GEMM_SOURCES = ["gemm_bf16.hip", "gemm_wgrad.hip", "decode.hip", "mx_gemm.hip"]

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")


def _remarks(src, tmp_path):
    from grouped_gemm_router_amd import build
    hipcc = build.HIPCC
    cmd = [hipcc, *build.FLAGS, "-c", os.path.join(CSRC, src), "-o", str(tmp_path / (src + ".o")),
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels = {}
    name = None
    for line in r.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            kernels[name] = {}
            continue
        m = re.search(r"remark:\s+(VGPRs Spill|SGPRs Spill|ScratchSize \[bytes/lane\]): (\d+)", line)
        if m and name:
            kernels[name][m.group(1)] = int(m.group(2))
    return kernels


@pytest.mark.parametrize("src", GEMM_SOURCES)
def test_gemm_kernels_do_not_spill(src, tmp_path):
    kernels = _remarks(src, tmp_path)
    assert kernels, "no kernel resource remarks"
    for name, res in kernels.items():
        assert res.get("VGPRs Spill", 0) == 0, (name, res)
        assert res.get("ScratchSize [bytes/lane]", 0) == 0, (name, res)
