"""Build-level checks (CPU): every hot kernel compiles for gfx950 with no
private-memory (scratch) use. A spilled accumulator tile or a parameter block
copied into private memory shows up here before it shows up as lost
throughput or extra HBM writes."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "comm_overlapped_linear_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", ["gemm.hip", "rowops.hip"])
def test_kernels_use_no_scratch(src, tmp_path):
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-c", os.path.join(CSRC, src),
           "-o", str(tmp_path / "k.o"), "-Rpass-analysis=kernel-resource-usage"]
    out = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stderr[-2000:]
    names = re.findall(r"Function Name: (\S+)", out.stderr)
    scratch = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", out.stderr)]
    assert names and len(names) == len(scratch)
    bad = [(n, s) for n, s in zip(names, scratch) if s != 0]
    assert not bad, bad
