"""The fp64 oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only) and driven through every code path by
tests/oracle_sanitize.c: recurrent form (all variants, windows, alignments,
feature maps, optional inputs, T = 0), decode steps, interpolation and
invalid arguments.  Any out-of-bounds access, leak or undefined operation
aborts the driver."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-D_GNU_SOURCE", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(ROOT, "oracle", "falcon_oracle.c"), os.path.join(HERE, "oracle_sanitize.c"),
           "-o", exe, "-lm", "-pthread"]
    subprocess.check_call(cmd)
    # verify_asan_link_order=0: a preloaded library may come before the ASan
    # runtime in the process's library list
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "oracle paths ok" in r.stdout
