"""Build the gfx950 HIP library ``libmoe_gfx950.so`` in-tree with hipcc, and
the benchmark's read-stream probe ``libmoe_probe_gfx950.so``."""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_gfx950.so")
PROBE_SRC = os.path.join(HERE, "probe", "read_stream.hip")
PROBE_LIB = os.path.join(HERE, "libmoe_probe_gfx950.so")
ROOT = os.path.dirname(HERE)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-result",
    # keep hipcc from emitting packed fp32 math (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed (%d): %s" % (res.returncode, " ".join(cmd)))


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every HIP source (in parallel) and link one shared library.
    Always recompiles."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in FLAGS if f != "-shared"]
    objs, cmds = [], []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".%d.o" % os.getpid())
        objs.append(obj)
        cmds.append([HIPCC, *compile_flags, "-c", src, "-o", obj])
    jobs = jobs or max(1, min(len(cmds), os.cpu_count() or 1, 16))
    tmp = LIB + ".tmp%d" % os.getpid()
    try:
        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
        os.replace(tmp, LIB)
    finally:
        # Objects are per build process; a failed build leaves none behind.
        for o in objs + [tmp]:
            if os.path.exists(o):
                os.remove(o)
    ptmp = PROBE_LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, *FLAGS, PROBE_SRC, "-o", ptmp], verbose)
    os.replace(ptmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
