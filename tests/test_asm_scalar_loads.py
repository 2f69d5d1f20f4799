"""The GEMV kernels read wave-uniform routing words with inline-asm scalar
loads (several in one block, waited for once).  A load's destination SGPR
must never be the address of another load of the same block: the data
returns asynchronously, so a later load could take a loaded value as its
address.  The outputs are early-clobber; this checks the compiled gfx950
assembly of every expert kernel instance (CPU only, needs hipcc)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_decode_gemv_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

LOAD = re.compile(r"s_load_dword s(\d+), s\[(\d+):(\d+)\]")


def asm_blocks(text):
    lines = text.splitlines()
    i = 0
    while i < len(lines):
        if "ASMSTART" in lines[i]:
            j = i + 1
            blk = []
            while "ASMEND" not in lines[j]:
                blk.append(lines[j].strip())
                j += 1
            yield blk
            i = j
        i += 1


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", ["experts_bf16.hip", "experts_fp8.hip", "experts_f32.hip", "experts_mfma.hip",
                                 "experts_mfma_wide.hip"])
def test_scalar_load_blocks_do_not_alias(tmp_path, src):
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
           os.path.join(CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    n = 0
    for blk in asm_blocks(out.read_text()):
        loads = [LOAD.match(l) for l in blk if l.startswith("s_load_dword ")]
        if not loads:
            continue
        n += 1
        outs = [int(m.group(1)) for m in loads]
        addrs = [{int(m.group(2)), int(m.group(3))} for m in loads]
        clash = [(a, b) for a in range(len(loads)) for b in range(len(loads)) if outs[a] in addrs[b]]
        assert not clash, "%s: load destination is another load's address: %s\n%s" % (src, clash, "\n".join(blk))
    if not src.startswith("experts_mfma"):
        assert n > 0
