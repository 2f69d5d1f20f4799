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
    # (buffer loads are the wide MFMA kernels' activation reads; spills would
    # be scratch accesses or buffer stores)
    assert not re.search(r"^\s*(scratch_(load|store)|buffer_store)", text, re.M), src


def _kernel_bodies(text, prefix):
    """{kernel name: its instruction lines} for the kernels whose names start with prefix;
    inline-asm blocks keep their #ASMSTART / #ASMEND markers."""
    out = {}
    for m in re.finditer(r"^(%s\w*):" % re.escape(prefix), text, re.M):
        end = text.index(".Lfunc_end", m.end())
        lines = []
        for l in text[m.end():end].split("\n"):
            l = l.strip()
            if l.startswith(";;#ASMSTART") or l.startswith(";;#ASMEND"):
                lines.append(l[2:])
                continue
            l = l.split(";")[0].strip()
            if l and not l.startswith("."):
                lines.append(l)
        out[m.group(1)] = lines
    return out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_narrow_mfma_ring_is_not_drained(tmp_path):
    """The narrow MFMA kernels wait for their LDS copies only through their
    own waits: the counted stage waits (s_waitcnt vmcnt(N) then s_barrier, in
    one asm block) and, once per item, an asm s_waitcnt vmcnt(0) for the
    item's route-id copy and fp8 scales, placed where all the previous item's
    copies have completed (one for the first item, one for each next item).
    A compiler wait on a vector load (e.g. the fp8 block scales) inside the
    stage loop would count without the copies and so drain the ring there; a
    compiler wait is allowed only right before an item wait, with no load or
    MFMA between them."""
    out = tmp_path / "experts_mfma.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
           os.path.join(CSRC, "experts_mfma.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    bodies = _kernel_bodies(out.read_text(), "_ZN3moe11mfma_kernel")
    assert len(bodies) == 8, sorted(bodies)  # bf16, fp8, MXFP4, q4_0 x two passes
    for name, lines in bodies.items():
        in_asm, block = [], None
        for l in lines:
            if l == "#ASMSTART":
                block = []
            elif l == "#ASMEND":
                block = None
            elif block is not None:
                block.append(l)
            in_asm.append(block is not None and l not in ("#ASMSTART", "#ASMEND"))
        item_waits = [i for i, l in enumerate(lines)
                      if l == "s_waitcnt vmcnt(0)" and in_asm[i] and lines[i - 1] == "#ASMSTART"
                      and lines[i + 1] == "#ASMEND"]
        assert len(item_waits) == 2, "%s: item waits at %s" % (name, item_waits)
        first = next(i for i, l in enumerate(lines) if l.startswith("global_load_lds"))
        last = max(i for i, l in enumerate(lines) if l.startswith("v_mfma"))
        for i in range(first, last):
            l = lines[i]
            if not (l.startswith("s_waitcnt") and "vmcnt" in l) or i in item_waits:
                continue
            if in_asm[i]:
                assert lines[i + 1] == "s_barrier", "%s: %s inside the stage loop" % (name, l)
                continue
            nxt = next((j for j in item_waits if j > i), None)
            assert nxt is not None and nxt - i <= 12, "%s: compiler wait %s at %d" % (name, l, i)
            between = lines[i + 1:nxt]
            assert not any(b.startswith(("global_load", "buffer_load", "v_mfma")) for b in between), \
                "%s: compiler wait %s at %d" % (name, l, i)
