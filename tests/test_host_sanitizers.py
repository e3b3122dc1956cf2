"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The host mirror of the planners (mla_plan_host.h, the code behind
mla_plan_host / mla_plan_groups_host) is built with g++ and both sanitizers
and fed random and adversarial call shapes (tests/sanitize/plan_fuzz.cpp).
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_latent_attention_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "sanitize", "plan_fuzz.cpp")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_planner_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "plan_fuzz")
    build = subprocess.run(
        ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-I", CSRC, SRC, "-o", exe],
        capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert run.stdout.strip() == "ok"
