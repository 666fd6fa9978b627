"""The forward-pass planner on the host: random shapes through
make_fwd_plan (compiled with g++ from la_abi.cpp, launchers stubbed) keep the
plan's invariants; no GPU needed."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_attention_attn_amd", "csrc")


def test_plan_invariants(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path / "plan_check")
    subprocess.check_call([gxx, "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                           os.path.join(ROOT, "tests", "plan_check.cpp"),
                           os.path.join(CSRC, "la_abi.cpp"), "-o", exe])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr


def test_plan_invariants_under_sanitizers(tmp_path):
    """The same host code (planner, argument checks) built for the host only
    with AddressSanitizer and UndefinedBehaviorSanitizer, every report fatal."""
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path / "plan_check_san")
    flags = ["-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    subprocess.check_call([gxx] + flags + ["-I", os.path.join(ROOT, "include"), "-I", CSRC,
                                           os.path.join(ROOT, "tests", "plan_check.cpp"),
                                           os.path.join(CSRC, "la_abi.cpp"), "-o", exe])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
