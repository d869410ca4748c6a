"""Pins for the oracle's amax and scale state (CPU only).

* The ring is checked against the closed form "maximum over the last
  min(n, 16) forwards", computed here by slicing a plain history list.
* The float32 divisions are checked against exact rational arithmetic
  (fractions.Fraction, rounded to float32 by a routine written here) and
  against a float64-divide-then-round route.
* The page's scale-file example (tests/golden/scale_file_example.json) gives
  exact static scales for two of its entries.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import AMAX_FLOOR, HISTORY_LEN, ScaleState, amax, scales_from_amax, static_amax_eff

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "scale_file_example.json")


def round_fraction_to_f32(fr: Fraction) -> np.float32:
    """Exact rational -> nearest float32 (ties to even), normal range only."""
    assert fr > 0
    e = fr.numerator.bit_length() - fr.denominator.bit_length()
    while Fraction(2) ** e > fr:
        e -= 1
    while Fraction(2) ** (e + 1) <= fr:
        e += 1
    assert -126 <= e <= 127
    scaled = fr / Fraction(2) ** (e - 23)          # in [2^23, 2^24)
    m = scaled.numerator // scaled.denominator
    rem = scaled - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    return np.float32(float(Fraction(m) * Fraction(2) ** (e - 23)))


def test_amax_basic():
    x = np.array([[0.5, -3.25], [2.0, 1.0]], dtype=np.float32)
    assert amax(x) == np.float32(3.25)
    assert amax(np.zeros((4, 4), np.float32)) == 0
    assert amax(np.zeros((0,), np.float32)) == 0
    assert amax(np.array([-0.0, -1e-30], np.float32)) == np.float32(1e-30)


def test_ring_closed_form():
    rng = np.random.default_rng(1)
    hist = []
    st = ScaleState()
    for n in range(1, 41):
        obs = rng.uniform(0.1, 10.0, 3).astype(np.float32)
        if n == 1:
            obs[:] = 1000.0       # a large first observation that must leave the window at n = 17
        hist.append(obs)
        st.forward_dynamic(obs)
        window = np.array(hist[max(0, n - HISTORY_LEN):n])
        want = window.max(axis=0)
        assert np.array_equal(st.amax_eff, want), n
        if 2 <= n <= 16:
            assert np.all(st.amax_eff == 1000.0)
        if n >= 17:
            assert np.all(st.amax_eff < 1000.0)


@pytest.mark.parametrize("hl", [1, 2, 5, 16])
def test_ring_history_lengths(hl):
    rng = np.random.default_rng(hl)
    st = ScaleState(history_len=hl)
    hist = []
    for n in range(1, 3 * hl + 3):
        obs = rng.uniform(0, 5, 3).astype(np.float32)
        hist.append(obs)
        st.forward_dynamic(obs)
        assert np.array_equal(st.amax_eff, np.array(hist[max(0, n - hl):n]).max(axis=0))


def test_bad_history_len():
    for hl in (0, 17, -1):
        with pytest.raises(ValueError):
            ScaleState(history_len=hl)


def test_scales_exact_rational_sample():
    for a in [1.0, 3.0, 7.0, 0.1, 1234.5, 2.0 ** -90, 448.0, 65504.0, 3.0e38]:
        a32 = np.float32(a)
        d, i = scales_from_amax(np.array([a32]))
        assert d[0] == round_fraction_to_f32(Fraction(float(a32)) / 448)
        if float(a32) > 2.0 ** -119:
            assert i[0] == round_fraction_to_f32(Fraction(448) / Fraction(float(a32)))


def test_scales_every_positive_bf16_amax():
    """All positive finite bf16 values as amax: float32 division equals float64 division rounded once.

    a/448 = a/(7*2^6): the exact quotient has a period-3 binary expansion, so it
    never lies within 2^-53 of a float32 midpoint and the float64 route cannot
    double-round differently.
    """
    bits = (np.arange(1, 0x7F80, dtype=np.uint32) << 16).view(np.float32)
    d, i = scales_from_amax(bits)
    a = np.maximum(bits, AMAX_FLOOR).astype(np.float64)
    assert np.array_equal(d, (a / 448.0).astype(np.float32))
    with np.errstate(over="ignore"):
        assert np.array_equal(i, (448.0 / a).astype(np.float32))
    fin = np.isfinite(i)
    assert fin[bits >= 2.0 ** -100].all()
    # inv * descale is 1 up to two roundings
    prod = i[fin].astype(np.float64) * d[fin].astype(np.float64)
    assert np.all(np.abs(prod - 1.0) < 2.0 ** -22)


def test_floor_for_zero_and_tiny():
    d, i = scales_from_amax(np.array([0.0, 2.0 ** -120], dtype=np.float32))
    assert np.all(np.isfinite(d)) and np.all(np.isfinite(i)) and np.all(d > 0)
    assert i[0] == np.float32(7 * 2.0 ** 106)          # 448 * 2^100 exactly
    assert d[0] == round_fraction_to_f32(Fraction(1, 448) / Fraction(2) ** 100)
    assert d[1] == d[0] and i[1] == i[0]


def test_static_mode_ignores_observed_and_keeps_ring():
    st = ScaleState(static_amax=[10.0, 20.0, 30.0], margin=1.5)
    d1, i1 = st.forward_static()
    assert np.array_equal(st.amax_eff, np.array([15.0, 30.0, 45.0], np.float32))
    assert np.all(st.ring == 0) and st.cursor == 0
    d2, _ = st.forward_static()
    assert np.array_equal(d1, d2)
    for t, a in enumerate([15.0, 30.0, 45.0]):
        assert d1[t] == round_fraction_to_f32(Fraction(a) / 448)
        assert i1[t] == round_fraction_to_f32(Fraction(448) / Fraction(a))


def test_static_margin_is_one_float32_multiply():
    sa = np.array([0.1, 3.3, 77.7], np.float32)
    m = np.float32(1.5)
    eff = static_amax_eff(sa, m)
    for t in range(3):
        assert eff[t] == round_fraction_to_f32(Fraction(float(sa[t])) * Fraction(float(m)))


def test_static_validation():
    for bad in ([1.0, 2.0], [1.0, -2.0, 3.0], [1.0, float("nan"), 3.0], [0.0, 1.0, 1.0]):
        with pytest.raises(ValueError):
            ScaleState(static_amax=bad)
    for m in (0.0, -1.0, float("inf")):
        with pytest.raises(ValueError):
            ScaleState(static_amax=[1.0, 1.0, 1.0], margin=m)
    with pytest.raises(ValueError):
        ScaleState(static_amax=[3e38, 1.0, 1.0], margin=1.5)     # product overflows float32
    with pytest.raises(ValueError):
        ScaleState().forward_static()


def test_scale_file_example_from_page():
    g = json.load(open(GOLDEN))
    entries = g["scales"]
    for layer, sc in entries.items():
        st = ScaleState(static_amax=[sc["q"], sc["k"], sc["v"]], margin=1.0)
        d, i = st.forward_static()
        for t, key in enumerate("qkv"):
            a = Fraction(sc[key])
            assert d[t] == round_fraction_to_f32(a / 448)
            assert i[t] == round_fraction_to_f32(Fraction(448) / a)
        for key, exp in g["exact"].get(layer, {}).items():
            t = "qkv".index(key)
            if "descale" in exp:
                assert d[t] == np.float32(exp["descale"])
            if "inv" in exp:
                assert i[t] == np.float32(exp["inv"])


def test_export_is_max_of_last_window_times_margin():
    """Calibration export = max of the last history_len observations x margin, one float32 multiply.

    Brute force over the list of observations (not the ring): checks the slot
    arithmetic of the ring, the wrap after history_len forwards and the single
    rounding of the margin product.
    """
    rng = np.random.default_rng(77)
    for hist in (16, 3, 1):
        st = ScaleState(history_len=hist)
        seen = [[], [], []]
        for n in range(1, 41):
            obs = (rng.uniform(0.5, 2.0, 3) * 2.0 ** rng.integers(-20, 20, 3)).astype(np.float32)
            st.forward_dynamic(obs)
            for t in range(3):
                seen[t].append(obs[t])
            for margin in (1.5, 1.0, 1.1):
                got = st.export_static_amax(margin)
                for t in range(3):
                    window = seen[t][max(0, n - hist):n]
                    want = round_fraction_to_f32(Fraction(float(max(window))) * Fraction(float(np.float32(margin))))
                    assert got[t] == want, (hist, n, t, margin)


def test_export_refusals():
    with pytest.raises(ValueError):
        ScaleState().export_static_amax(1.5)                 # nothing observed yet
    st = ScaleState()
    st.forward_dynamic([1.0, 0.0, 1.0])
    with pytest.raises(ValueError):
        st.export_static_amax(1.5)                           # V observed only zeros
    st = ScaleState()
    st.forward_dynamic([3e38, 1.0, 1.0])
    with pytest.raises(ValueError):
        st.export_static_amax(1.5)                           # product overflows float32
    for m in (0.0, -1.0, float("nan")):
        with pytest.raises(ValueError):
            st.export_static_amax(m)


def test_export_then_load_equals_margin_at_load():
    """fp32(fp32(a * m) * 1) == fp32(a * m): saving with the margin and loading with margin 1.0
    gives the same scales as loading the raw ring maximum with the margin."""
    st = ScaleState()
    for obs in ([224.3, 0.7, 13.0], [100.0, 1.9, 12.5], [3.3, 0.2, 99.0]):
        st.forward_dynamic(np.array(obs, np.float32))
    saved = st.export_static_amax(1.5)
    a = ScaleState(static_amax=saved, margin=1.0)
    b = ScaleState(static_amax=st.ring.max(axis=1), margin=1.5)
    da, ia = a.forward_static()
    db, ib = b.forward_static()
    assert np.array_equal(da, db) and np.array_equal(ia, ib)
