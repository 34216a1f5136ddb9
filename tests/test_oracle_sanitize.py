"""The oracle under the host sanitizers: tests/oracle_sanitize_main.c calls
every oracle entry point on small ragged shapes, built with
-fsanitize=address,undefined (and -fno-sanitize-recover, so any report fails)."""
import os
import shutil
import subprocess

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = tmp_path / "oracle_sanitize"
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", oracle.SOURCE,
           os.path.join(HERE, "oracle_sanitize_main.c"), "-o", str(exe), "-lm", "-lpthread"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout
