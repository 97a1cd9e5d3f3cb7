"""The host planner under the address and undefined-behaviour sanitizers.

tests/sanitize/plan_fuzz.cpp drives the planner with random configurations and
batches (single format and shared-prefix compositions) and checks the structure
of every plan blob; every other case is planned a second time with its chunking
candidates scored on threads, which must give the same bytes.  It is compiled
here with g++ (host code only, no HIP) and run; a sanitizer report or a failed
check fails the test.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "serving_attention_bsr_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_planner_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "plan_fuzz")
    cmd = [
        "g++", "-std=c++17", "-O1", "-g", "-pthread", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
        "-fno-omit-frame-pointer", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
        os.path.join(ROOT, "tests", "sanitize", "plan_fuzz.cpp"), os.path.join(CSRC, "plan.cpp"), "-o", exe,
    ]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    # (verify_asan_link_order=0: the environment may preload another library first)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    proc = subprocess.run([exe, "1500", "7"], capture_output=True, text=True, env=env, timeout=600)
    assert proc.returncode == 0, proc.stdout + proc.stderr
    assert "runtime error" not in proc.stderr, proc.stderr
    assert "planned" in proc.stdout
