"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer
(host only): tests/sanitize/oracle_main.c drives every C entry point on
exact-size heap buffers, so a read or write past a tensor or undefined index
arithmetic aborts the run."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-Wno-unknown-pragmas", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fopenmp", os.path.join(ROOT, "oracle", "oracle.c"),
           os.path.join(HERE, "sanitize", "oracle_main.c"), "-lm", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1"))
    out = r.stdout + r.stderr
    assert r.returncode == 0, out
    assert "OK" in r.stdout and "runtime error" not in out and "AddressSanitizer" not in out, out
