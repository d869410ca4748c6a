"""Compile the HIP sources into quantized_flash_attn_amd/libqfa.so (gfx950 only).

Run ``python quantized_flash_attn_amd/build.py`` (or ``__graft_entry__.build()``).
Run it as a script, not as ``-m quantized_flash_attn_amd.build``: importing the
package loads the library, which is missing before the first build.
hipcc cross-compiles for gfx950 without a GPU present.
"""

import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libqfa.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["abi.hip", "quant.hip", "attn.hip", "attn_bf16.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 instructions stay disabled on the device
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = [ln for ln in res.stdout.splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("build failed:\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines), flush=True)


# Test infrastructure built alongside the library: a one-wave probe of the
# matrix instructions' summation (tests/test_gpu_mfma_hw.py loads it), and a
# full-chip matrix-throughput kernel (bench.py --power).  Its matrix
# instructions write their accumulators to ordinary VGPRs, so the throughput
# loop carries no accumulator copies.
PROBE_SRC = os.path.join(ROOT, "tests", "hw", "mfma_probe.hip")
PROBE_LIB = os.path.join(ROOT, "tests", "hw", "libmfma_probe.so")


def build_probe(verbose: bool = True) -> str:
    """Compile the test-side MFMA probe library; return its path."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="qfa_probe_") as tmp:
        out = os.path.join(tmp, "libmfma_probe.so")
        _run([cc, *HIPCC_FLAGS, "-mllvm", "-amdgpu-mfma-vgpr-form=1", "-shared", PROBE_SRC, "-o", out], verbose)
        shutil.copyfile(out, PROBE_LIB + ".tmp")
        os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return PROBE_LIB


def build(verbose: bool = True) -> str:
    """Compile every source and link the shared library; return its path."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="qfa_build_") as tmp:
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            _run([cc, *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
            objs.append(obj)
        tmp_lib = os.path.join(tmp, LIB_NAME)
        _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp_lib], verbose)
        shutil.copyfile(tmp_lib, LIB_PATH + ".tmp")
        os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
    build_probe(verbose="-q" not in sys.argv)
