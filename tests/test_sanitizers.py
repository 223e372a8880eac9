"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer: the planner (plan.cpp, built
with g++ on its own, no GPU code) and the C oracle, each driven over seeded random and malformed
inputs by a small driver in tests/sanitize/.  Any sanitizer report makes the driver exit non-zero."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd_build, exe, tmp_path):
    r = subprocess.run(cmd_build, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env, cwd=str(tmp_path))
    assert r.returncode == 0 and r.stdout.startswith("OK"), (r.stdout[-2000:], r.stderr[-4000:])
    return r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_planner_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "plan_driver")
    out = _run(["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"),
                os.path.join(HERE, "plan_driver.cpp"),
                os.path.join(ROOT, "block_causal_chunk_amd", "csrc", "plan.cpp"), "-o", exe], exe, tmp_path)
    print(out)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", *SAN, "-fopenmp", os.path.join(HERE, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "wf_oracle.c"), "-o", exe, "-lm"], exe, tmp_path)
