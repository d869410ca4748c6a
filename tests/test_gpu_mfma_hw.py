"""GPU: how gfx950's matrix instructions sum products (hardware pins for the kernel design).

The E4M3 attention kernel converts codes to fp16 and multiplies on the fp16
MFMA instead of the fp8 MFMAs.  This test pins the two facts that choice
rests on, with one wave running one instruction (tests/hw/mfma_probe.hip) on
operands whose lane 0 holds K elements 0..7 of row 0 of A and column 0 of B
(all other elements zero), so output element (0, 0) in lane 0 is
c + sum_k a_k b_k over one group of 8 consecutive products:

* the fp8 MFMAs (v_mfma_f32_16x16x128_f8f6f4 and v_mfma_f32_16x16x32_fp8_fp8)
  add a group of 8 products on a window of about 13 bits below the group's
  largest product and truncate the rest: 2^14 + 7 * 1 comes out as 2^14, and
  2^11 + 7 * 0.875 as 2^11 + 7 * 0.75.  Each product is cut to a multiple of
  2^(E - 13), E the exponent of the group's largest product, toward zero
  (2^11 - 7 * 0.875 gives 2^11 - 7 * 0.75).  The accumulator input is added
  to the group's sum exactly (65536 + 7 stays 65543);
* the fp16 and bf16 MFMAs return the exact sums (every product of two E4M3
  values has at most 8 significant bits, and these sums fit fp32).

With x20 outliers in both Q and K, a query and key sharing an outlier
dimension have a product near 2^13-2^17 in one group, so the fp8 MFMAs would
truncate the other 7 products of that group and move dominant logits
(tests/test_fp8_mfma_emulation.py works out what that does to the
workloads' attention on the CPU).
"""

import ctypes
import os

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hw", "libmfma_probe.so")
KIND = {"f8f6f4_k128": 0, "fp8_k32": 1, "f16_k32": 2, "bf16_k32": 3}


def _lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB)
    lib.mfma_probe.restype = ctypes.c_int
    lib.mfma_probe.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 5
    return lib


def _lane0_bytes(kind, vals):
    """Register image of lane 0 holding vals as K elements 0..len(vals)-1."""
    vals = np.asarray(vals, dtype=np.float32)
    if kind in ("f8f6f4_k128", "fp8_k32"):
        c = oracle.encode(vals)
        assert np.array_equal(oracle.decode(c), vals), "probe values must be E4M3 values"
        return c.tobytes()
    if kind == "f16_k32":
        return vals.astype(np.float16).tobytes()
    return torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().tobytes()


def run_probe(kind, a_vals, b_vals, c00=0.0):
    lib = _lib()
    a = np.zeros(64 * 32, np.uint8)
    b = np.zeros(64 * 32, np.uint8)
    ab, bb = _lane0_bytes(kind, a_vals), _lane0_bytes(kind, b_vals)
    a[:len(ab)] = np.frombuffer(ab, np.uint8)
    b[:len(bb)] = np.frombuffer(bb, np.uint8)
    c = np.zeros(64 * 4, np.float32)
    c[0] = c00
    da, db = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    dc = torch.from_numpy(c).cuda()
    dd = torch.empty_like(dc)
    st = torch.cuda.current_stream().cuda_stream
    assert lib.mfma_probe(KIND[kind], da.data_ptr(), db.data_ptr(), dc.data_ptr(), dd.data_ptr(), st) == 0
    torch.cuda.synchronize()
    d = dd.cpu().numpy()
    others = np.delete(d, 0)
    assert np.all(others == 0.0), "only element (0, 0) has non-zero products"
    return float(d[0])


CASES = [
    # (name, a values, b values, accumulator in, exact sum)
    ("2^14 + 7 x 1", [128.0] + [1.0] * 7, [128.0] + [1.0] * 7, 0.0, 16391.0),
    ("2^11 + 7 x 0.875", [64.0] + [0.875] * 7, [32.0] + [1.0] * 7, 0.0, 2054.125),
    ("65536 acc + 7", [7.0], [1.0], 65536.0, 65543.0),
    ("2^11 - 7 x 0.875", [64.0] + [-0.875] * 7, [32.0] + [1.0] * 7, 0.0, 2041.875),
]

# What gfx950 returns for the fp8 instructions: truncated group sums, exact accumulator add.
FP8_OBSERVED = {
    "f8f6f4_k128": [16384.0, 2053.25, 65543.0, 2042.75],
    "fp8_k32": [16384.0, 2053.25, 65543.0, 2042.75],
}


@pytest.mark.parametrize("kind", ["f16_k32", "bf16_k32"])
def test_16bit_mfma_sums_exactly(kind):
    for name, a, b, c00, exact in CASES:
        got = run_probe(kind, a, b, c00)
        print(f"{kind} {name}: {got!r} (exact {exact!r})", flush=True)
        assert got == exact, (kind, name, got, exact)


@pytest.mark.parametrize("kind", ["f8f6f4_k128", "fp8_k32"])
def test_fp8_mfma_truncates_inside_a_group(kind):
    for (name, a, b, c00, exact), want in zip(CASES, FP8_OBSERVED[kind]):
        got = run_probe(kind, a, b, c00)
        print(f"{kind} {name}: {got!r} (exact {exact!r})", flush=True)
        assert got == want, (kind, name, got, want)
    # the truncation is what makes the fp8 sum differ from the exact one
    assert run_probe(kind, *CASES[0][1:4]) != CASES[0][4]
