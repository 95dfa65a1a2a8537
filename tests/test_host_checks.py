"""Host-side argument checks: g++ unit test (ASan + UBSan) of mla_host_checks.h."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_checks_with_sanitizers(tmp_path):
    exe = tmp_path / "host_checks_test"
    src = os.path.join(HERE, "native", "host_checks_test.cpp")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-Wall", "-Wextra", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", src, "-o", str(exe)]
    subprocess.run(cmd, check=True)
    res = subprocess.run([str(exe)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert res.returncode == 0, res.stdout
    assert "host checks OK" in res.stdout
