"""The call-epoch rule of a workspace (poisoning after a bounded wait gives up) and the
arrival that ends a call, built for the host from the same header the kernels include and
run with threads standing in for workgroups."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "draft_verification_softmax_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "cpp", "epoch_rule_test.cc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_epoch_rule_and_arrival(tmp_path):
    exe = str(tmp_path / "epoch_rule_test")
    subprocess.run(["g++", "-std=c++17", "-O1", "-pthread", "-Wall", "-Werror", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-I", CSRC, "-o", exe, SRC], check=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.strip().endswith("ok")
