"""Pins for the oracle's quantizer (CPU only).

* With a power-of-two factor the float32 product is exact, so the codes must
  equal torch-CPU's own float8_e4m3fn cast of the scaled values.
* Dequantization error bound: ``|decode(code) * descale - x|`` is at most half
  an E4M3 spacing of ``x * inv`` times ``descale`` (catches a swapped inv /
  descale or a dropped scale).
* On a forward whose own amax sets the scale, the largest element maps to 448.
"""

import numpy as np
import torch

from oracle import ScaleState, decode, quantize, quantize_qkv
from workloads import WORKLOADS, make_qkv


def _f32(t):
    return t.float().numpy()


def test_power_of_two_factor_matches_torch_cast():
    q, _, _ = make_qkv(WORKLOADS[1], 0)
    x = _f32(q)
    for inv in (1.0, 4.0, 2.0 ** -3, 32.0):
        codes = quantize(x, np.float32(inv))
        y = torch.from_numpy(np.clip(x * np.float32(inv), -448, 448)).to(torch.float8_e4m3fn)
        assert np.array_equal(codes, y.view(torch.uint8).numpy())


def test_dynamic_forward_error_bound_and_max_code():
    w = WORKLOADS[1]
    st = ScaleState()
    for fwd in range(3):
        q, k, v = (_f32(t) for t in make_qkv(w, fwd))
        q8, k8, v8, descale, observed = quantize_qkv(st, "dynamic", q, k, v)
        for x, c, d, obs in zip((q, k, v), (q8, k8, v8), descale, observed):
            assert obs == np.abs(x).max()
            back = decode(c) * np.float64(d)
            a = np.abs(x.astype(np.float64)) / np.float64(d)           # |x| in code units
            spacing = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 1e-300))) - 3))
            tol = (spacing / 2) * np.float64(d) * (1 + 1e-6) + np.abs(x) * 2.0 ** -22
            assert np.all(np.abs(back - x) <= tol)
        if fwd == 0:
            # the first forward's scale comes from its own amax: the max element encodes to +-448
            for c in (q8, k8, v8):
                assert (c & 0x7F).max() == 0x7E


def test_static_mode_saturates_when_data_exceeds_scale():
    w = WORKLOADS[1]
    q, k, v = (_f32(t) for t in make_qkv(w, 0))
    st = ScaleState(static_amax=[1.0, 1.0, 1.0], margin=1.0)   # far below the data's range (outliers x30)
    q8, k8, v8, descale, _ = quantize_qkv(st, "static", q, k, v)
    assert np.all(descale == np.float32(1.0 / 448.0))
    big = np.abs(q) >= 1.0
    assert big.any() and np.all((q8[big] & 0x7F) == 0x7E)
    assert np.all(st.ring == 0)


def test_zero_tensor_quantizes_to_zero():
    st = ScaleState()
    z = np.zeros((8, 2, 128), np.float32)
    q8, k8, v8, descale, _ = quantize_qkv(st, "dynamic", z, z, -z)
    assert np.all(q8 == 0) and np.all(k8 == 0) and np.all(v8 == 0x80)
    assert np.all(np.isfinite(descale)) and np.all(descale > 0)


def test_packed_quantize_brute_force():
    """Fused [T, 3, H, D] input: element by element, each code is encode(fp32(x * inv)) of its own tensor's
    scale at [t, h, d], dims past D are 0, and the amax counts only the tensor's own real elements."""
    from oracle import ScaleState, encode, quantize_qkv_packed

    rng = np.random.default_rng(12)
    T, H, D = 3, 2, 16
    qkv = rng.standard_normal((T, 3, H, D)).astype(np.float32) * np.array([1.0, 7.0, 0.25], np.float32)[None, :, None, None]
    qkv = qkv.astype(np.float32)
    q8, k8, v8, descale, observed = quantize_qkv_packed(ScaleState(), "dynamic", qkv)
    codes = (q8, k8, v8)
    for which in range(3):
        brute_amax = 0.0
        for t in range(T):
            for h in range(H):
                for d in range(D):
                    brute_amax = max(brute_amax, abs(float(qkv[t, which, h, d])))
        assert observed[which] == np.float32(brute_amax)
        inv = np.float32(448.0) / np.float32(max(brute_amax, 2.0 ** -100))
        for t in range(T):
            for h in range(H):
                for d in range(128):
                    want = 0 if d >= D else int(encode(np.array([np.float32(qkv[t, which, h, d]) * inv], np.float32))[0])
                    assert codes[which][t, h, d] == want, (which, t, h, d)
    assert descale.dtype == np.float32 and descale.shape == (3,)
