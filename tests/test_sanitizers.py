"""The host C code of the test infrastructure -- the CPU oracle and the seeded
input generator, both multi-threaded C with manual indexing -- built with
AddressSanitizer + UndefinedBehaviorSanitizer and with ThreadSanitizer and
driven through every entry point on small inputs (tests/sanitizer_driver.c).
Any out-of-bounds access, use after free, leak, undefined behaviour or data
race aborts the driver.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = [os.path.join(ROOT, "tests", "sanitizer_driver.c"), os.path.join(ROOT, "oracle", "moe_oracle.c"),
           os.path.join(ROOT, "workload", "moegen.c")]
GCC = shutil.which("gcc")

FLAVOURS = {
    "address_undefined": (["-fsanitize=address,undefined", "-fno-sanitize-recover=all"],
                          {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=1",
                           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}),
    "thread": (["-fsanitize=thread"], {"TSAN_OPTIONS": "halt_on_error=1"}),
}


@pytest.mark.skipif(GCC is None, reason="gcc not available")
@pytest.mark.parametrize("flavour", sorted(FLAVOURS))
def test_oracle_and_generator_under_sanitizer(tmp_path, flavour):
    flags, env_add = FLAVOURS[flavour]
    exe = tmp_path / ("driver_" + flavour)
    cmd = [GCC, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-pthread", "-fno-fast-math",
           "-ffp-contract=off", *flags, *SOURCES, "-o", str(exe), "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0 and "cannot find" in res.stderr:
        pytest.skip("sanitizer runtime not installed: " + res.stderr.strip()[:200])
    assert res.returncode == 0, res.stderr
    env = dict(os.environ, **env_add)
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "sanitizer driver ok" in run.stdout
