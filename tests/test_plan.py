"""Launch planning (pure C++ header) compiled with g++ and checked on the host:
bijection of workgroup ids, exact coverage of every query row, GQA head
mapping, causal tile counts, heavy-first order and the XCD remap."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


# host-only sanitizers (address, undefined behaviour incl. signed overflow)
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def test_plan_checks(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = tmp_path / "plan_check"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROOT, "exact_attention_07_amd", "csrc"),
           os.path.join(ROOT, "tests", "plan_check.cpp"), "-o", str(exe)]
    # with the sanitizers where their runtimes are installed, plain otherwise
    if subprocess.run(cmd[:1] + SANITIZE + cmd[1:], capture_output=True).returncode != 0:
        subprocess.run(cmd, check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "plan checks passed" in r.stdout
