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


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_abi_from_plain_c(tmp_path):
    """The header is plain C99 and the library links and answers from C."""
    root = os.path.dirname(HERE)
    lib_dir = os.path.join(root, "attention_mla_causal_amd")
    if not os.path.exists(os.path.join(lib_dir, "libmla_attn.so")):
        pytest.skip("library not built")
    exe = tmp_path / "abi_c_test"
    src = os.path.join(HERE, "native", "abi_c_test.c")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", src, "-o", str(exe),
           "-L" + lib_dir, "-lmla_attn", "-Wl,-rpath," + lib_dir]
    subprocess.run(cmd, check=True)
    res = subprocess.run([str(exe)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert res.returncode == 0, res.stdout
    assert "abi c OK" in res.stdout
