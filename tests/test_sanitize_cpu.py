"""Host sanitizer builds: the planner (csrc/plan.cpp, the library's host
half) and the oracle (oracle/oracle.c), each compiled with gcc's
AddressSanitizer and UndefinedBehaviorSanitizer into a driver executable of
its own and run over random and edge-case arguments.  A sanitizer report
(out-of-bounds access, leak, signed overflow, bad shift, ...) or a non-zero
exit fails the test.  Host code only: no GPU code is built here."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=24")


def _build_and_run(tmp_path, compiler, sources, extra):
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not found")
    exe = str(tmp_path / "driver")
    cmd = [compiler, *SAN, *extra, *sources, "-lm", "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0 and "asan" in (res.stderr or "").lower():
        pytest.skip("no sanitizer runtime: " + res.stderr[-300:])
    assert res.returncode == 0, " ".join(cmd) + "\n" + res.stderr[-3000:]
    env = dict(ENV)
    env.pop("LD_PRELOAD", None)  # the sanitizer runtime must come first
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    report = run.stdout[-2000:] + run.stderr[-4000:]
    assert run.returncode == 0, report
    assert "runtime error" not in run.stderr and "Sanitizer" not in run.stderr, report
    assert "driver done" in run.stdout, report


def test_planner_under_asan_ubsan(tmp_path):
    csrc = os.path.join(ROOT, "vision_image_preprocessing_amd", "csrc")
    _build_and_run(tmp_path, "g++",
                   [os.path.join(HERE, "plan_driver.cpp"), os.path.join(csrc, "plan.cpp")],
                   ["-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", csrc])


def test_oracle_under_asan_ubsan(tmp_path):
    _build_and_run(tmp_path, "gcc",
                   [os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "oracle.c")],
                   ["-std=c11", "-ffp-contract=off"])
