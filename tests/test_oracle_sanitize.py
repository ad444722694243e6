"""The C oracle under gcc's AddressSanitizer and UndefinedBehaviorSanitizer.

tests/oracle_sanitize_main.c drives every oracle entry point over ragged and
degenerate shapes (count 0, 1, 59..61, 119..121, 4099; 1 to 16 ranks), every
protocol and epochs next to the wrap, from exact-size heap buffers; it also
checks round trips, corrupt flags and two-shot == one-shot bit for bit.  Host
code only: nothing here touches a GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "ar_oracle.c")
DRIVER_C = os.path.join(ROOT, "tests", "oracle_sanitize_main.c")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    build = subprocess.run(
        ["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
         ORACLE_C, DRIVER_C, "-o", exe, "-lm"],
        capture_output=True, text=True, timeout=300)
    if build.returncode != 0 and "sanitize" in build.stderr:
        pytest.skip("gcc has no sanitizer runtime here: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "0 failures" in run.stdout
