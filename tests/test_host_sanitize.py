"""Host code under gcc's AddressSanitizer and UndefinedBehaviorSanitizer: the
C oracle, and the library's cost-table selector (its only pure host file).

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


SELECT_CPP = os.path.join(ROOT, "collective_synchronization_amd", "csrc", "ar_select.cpp")
SELECT_DRIVER = os.path.join(ROOT, "tests", "select_sanitize_main.c")


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                    reason="needs gcc and g++")
def test_selector_under_address_and_undefined_sanitizers(tmp_path):
    """ar_select.cpp's three entry points: the documented argument errors, and
    48000 random choices against a brute-force reading of the rule in
    include/ar.h, from exact-size heap tables."""
    san = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer"]
    sel_o, drv_o, exe = (str(tmp_path / n) for n in ("sel.o", "drv.o", "select_sanitize"))
    for cmd in (["g++", "-std=c++17", *san, "-c", SELECT_CPP, "-o", sel_o],
                ["gcc", "-std=c11", *san, "-c", SELECT_DRIVER, "-o", drv_o],
                ["g++", "-fsanitize=address,undefined", sel_o, drv_o, "-o", exe, "-lm"]):
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
        if r.returncode != 0 and "sanitize" in r.stderr:
            pytest.skip("no sanitizer runtime here: " + r.stderr[-300:])
        assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "0 failures" in run.stdout
