"""Code-generation checks on the gfx950 assembly of every HIP source (CPU
only: hipcc cross-compiles).  The kernels are written to run without
function calls and without scratch memory: a call spills registers around
it, and scratch accesses are vector memory operations, so waiting for one
also waits for every weight load in flight."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_decode_gemv_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", SOURCES)
def test_no_calls_no_scratch(tmp_path, src):
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
           os.path.join(CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    text = out.read_text()
    assert "s_swappc" not in text, "%s: a device function is called instead of inlined" % src
    sizes = [int(v) for v in re.findall(r"\.amdhsa_private_segment_fixed_size\s+(\d+)", text)]
    assert max(sizes, default=0) == 0, "%s: a kernel uses scratch memory" % src
    assert not re.search(r"^\s*(scratch|buffer)_(load|store)", text, re.M), src
