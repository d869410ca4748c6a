"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds a copy of the library whose host code (argument checks, status and
error text, size arithmetic, dispatch) is instrumented with ASan and UBSan
(the device code is built as usual, uninstrumented), then runs two C
programs linked against it, each instrumented too:

* tests/abi_c_check.c, the documented statuses of the argument checks;
* tests/abi_sweep.c, every entry point under edge and seeded random
  arguments, checking that each status is a declared code with an error
  text, and that nothing that would enqueue work succeeds.

Any out-of-bounds access, use after free, leak, signed overflow, invalid
enum load or other undefined behaviour aborts the program with a report.
Both programs pass placeholder device addresses, so they run only on a host
whose HIP runtime sees no GPU (the sweep checks this itself and exits early
otherwise).  No GPU needed.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_flash_attn_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
SOURCES = ["abi.hip", "quant.hip", "attn.hip", "attn_bf16.hip"]

# Host-only instrumentation: every sanitizer flag applies to the host pass.
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    assert res.returncode == 0, " ".join(cmd) + "\n" + res.stdout[-4000:]
    return res.stdout


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("hipcc / ROCm clang not available")
    d = tmp_path_factory.mktemp("qfa_san")
    procs = []
    for src in SOURCES:
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17", "-I", INCLUDE,
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SAN,
               "-c", os.path.join(CSRC, src), "-o", str(d / (src + ".o"))]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    for cmd, p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, " ".join(cmd) + "\n" + out[-4000:]
    lib = d / "libqfa_san.so"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_SAN[:4], "-shared-libsan",
          *[str(d / (s + ".o")) for s in SOURCES], "-o", str(lib)])
    runtime = os.path.join(_run([CLANG, "-print-resource-dir"]).strip(), "lib", "linux")
    if not os.path.exists(os.path.join(runtime, "libclang_rt.asan-x86_64.so")):
        pytest.skip("clang ASan runtime not found")
    exes = {}
    for name in ("abi_c_check", "abi_sweep"):
        exe = str(d / name)
        _run([CLANG, "-std=c99", "-g", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
              "-I", os.path.join(ROCM, "include"), "-I", INCLUDE, "-fsanitize=address,undefined",
              "-fno-sanitize-recover=all", "-shared-libsan", os.path.join(ROOT, "tests", name + ".c"),
              "-L", str(d), "-lqfa_san", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
              "-Wl,-rpath," + str(d), "-Wl,-rpath," + runtime, "-Wl,-rpath," + os.path.join(ROCM, "lib"),
              "-o", exe])
        exes[name] = exe
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return exes, env


def test_documented_statuses_under_sanitizers(sanitized):
    exes, env = sanitized
    out = _run([exes["abi_c_check"]], env=env, timeout=120)
    assert "C ABI checks ok" in out, out


def test_argument_sweep_under_sanitizers(sanitized):
    exes, env = sanitized
    out = _run([exes["abi_sweep"]], env=env, timeout=300)
    if "a GPU is present" in out:
        pytest.skip("the sweep runs only where the HIP runtime sees no GPU")
    assert "ABI sweep ok" in out, out
