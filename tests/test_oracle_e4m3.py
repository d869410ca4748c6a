"""Pins for the oracle's E4M3 codec (CPU only).

The codec is pinned to things outside itself: the OCP format's named points
(tests/golden/ocp_e4m3_points.txt), torch-CPU's independent float8_e4m3fn
implementation over every bf16 input, and tie cases derived by hand from the
round-to-nearest-even rule.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import DECODE_TABLE, decode, encode

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ocp_e4m3_points.txt")


def _all_bf16_as_f32():
    bits = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    return bits[~np.isnan(bits)]


def _torch_encode(y32):
    """torch-CPU float32 -> float8_e4m3fn after a +-448 clamp (torch's cast does not saturate)."""
    t = torch.from_numpy(np.clip(y32, -448.0, 448.0).astype(np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_golden_points():
    n = 0
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        code_s, value_s = line.split()[:2]
        code = int(code_s, 16)
        value = float(value_s)
        got = DECODE_TABLE[code]
        if math.isnan(value):
            assert math.isnan(got)
        else:
            assert got == value and math.copysign(1.0, got) == math.copysign(1.0, value)
        n += 1
    assert n >= 10


def test_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(encode(decode(codes).astype(np.float32)), codes)


@pytest.mark.parametrize("scale", [1.0, 2.0 ** -7, 2.0 ** 3, 64.0, 448.0 / 3.0, 448.0 / 7.5, 448.0 / 301.0, 0.37])
def test_encode_matches_torch_every_bf16(scale):
    x = _all_bf16_as_f32()
    with np.errstate(over="ignore"):
        y = (x * np.float32(scale)).astype(np.float32)
    assert np.array_equal(encode(y), _torch_encode(y))


@pytest.mark.parametrize(
    "y,code",
    [
        (1.0625, 0x38),             # halfway between 1.0 (m=0) and 1.125 (m=1): even -> 1.0
        (1.1875, 0x3A),             # halfway between 1.125 (m=1) and 1.25 (m=2): even -> 1.25
        (1.5 * 2.0 ** -9, 0x02),    # halfway between subnormals 1 and 2: even -> 2
        (0.5 * 2.0 ** -9, 0x00),    # halfway between 0 and the smallest subnormal: even -> 0
        (-0.5 * 2.0 ** -9, 0x80),   # same, negative: signed zero
        (-0.0, 0x80),
        (7.5 * 2.0 ** -9, 0x08),    # halfway between largest subnormal and smallest normal: even -> 2^-6
        (2.0 ** -6 * 1.0625, 0x08), # halfway above the smallest normal: even -> 2^-6
        (432.0, 0x7E),              # halfway between 416 and 448: even (m=6) -> 448
        (460.0, 0x7E),              # saturates
        (464.0, 0x7E),              # would round to 480: saturates
        (1e30, 0x7E),
        (float("inf"), 0x7E),
        (float("-inf"), 0xFE),
        (-448.0, 0xFE),
        (1e-30, 0x00),
    ],
)
def test_encode_ties_and_saturation(y, code):
    assert int(encode(np.array([y], dtype=np.float32))[0]) == code


def test_encode_rejects_nan():
    with pytest.raises(ValueError):
        encode(np.array([1.0, float("nan")], dtype=np.float32))


def test_encode_error_bound():
    """|decode(encode(y)) - y| is at most half a spacing, for random float32 inputs in range."""
    rng = np.random.default_rng(0)
    y = (rng.standard_normal(200000) * np.exp(rng.uniform(-14, 6, 200000))).astype(np.float32)
    y = np.clip(y, -448, 448)
    back = decode(encode(y))
    a = np.abs(y.astype(np.float64))
    spacing = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 1e-300))) - 3))
    assert np.all(np.abs(back - y) <= spacing / 2)
