"""The oracle under the address and undefined-behaviour sanitizers: every
entry point runs on small, ragged shapes with exact-size heap buffers
(tests/sanitize/oracle_drive.c), and any out-of-bounds access, bad shift,
overflow or misaligned access aborts the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "oracle_drive"
    cmd = ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-ffp-contract=off", "-Wno-unknown-pragmas",
           os.path.join(ROOT, "tests", "sanitize", "oracle_drive.c"),
           os.path.join(ROOT, "oracle", "bq8_oracle.c"), "-o", str(exe), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stderr[-4000:]
    assert r.stdout.strip() == "ok"
