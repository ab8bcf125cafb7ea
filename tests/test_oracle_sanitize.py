"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only) and run on small seeded inputs through every entry
point, error paths included (tests/oracle_sanitize_driver.c).  Any heap
overflow, use after free, leak or undefined behaviour aborts the driver."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "oracle_asan"
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-o", str(exe), os.path.join(HERE, "oracle_sanitize_driver.c"),
           os.path.join(ROOT, "oracle", "tev_oracle.c"), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=24", OMP_NUM_THREADS="2")
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert res.returncode == 0, f"rc {res.returncode}\n{res.stdout}\n{res.stderr[-4000:]}"
    assert "oracle sanitize driver ok" in res.stdout
