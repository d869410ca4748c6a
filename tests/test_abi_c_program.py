"""The C ABI from a plain C program (no Python, no torch, no GPU).

Compiles tests/abi_c_check.c as C99 with gcc against include/qfa.h, links it
against the built libqfa.so and runs it: the header must be valid C, every
declared entry point must link, and the argument checks (which return before
any HIP call) must give the documented statuses.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "quantized_flash_attn_amd")
LIB = os.path.join(PKG, "libqfa.so")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_program_uses_the_abi(tmp_path):
    assert os.path.exists(LIB), "libqfa.so is not built (run quantized_flash_attn_amd/build.py)"
    exe = str(tmp_path / "abi_c_check")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "abi_c_check.c"), "-L", PKG, "-lqfa", "-Wl,-rpath," + PKG, "-o", exe]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert res.returncode == 0, res.stdout
    run = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    assert run.returncode == 0 and "C ABI checks ok" in run.stdout, run.stdout
