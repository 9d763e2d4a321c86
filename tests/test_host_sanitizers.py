"""The host library's argument validation and launch planning (plan.cpp, pure
C++) built with AddressSanitizer and UndefinedBehaviorSanitizer and driven
with 20000 rounds of seeded random arguments (tests/sanitize/check_driver.cpp).
No GPU and no HIP runtime are involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_planning_and_checks_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = tmp_path / "check_driver"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", os.path.join(ROOT, "tests", "sanitize", "check_driver.cpp"),
           os.path.join(ROOT, "eagle_draft_tree_attention_amd", "csrc", "plan.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "0 plan inconsistencies" in r.stdout
