"""Pins for the oracle's varlen attention (CPU only).

* Library special case: when every input is an E4M3 value times 2^-6 and the
  largest magnitude is exactly 7, the scales are exact powers of two and
  quantization is lossless, so the oracle must equal torch-CPU's float64
  scaled_dot_product_attention on the original values, per sequence.
* Brute force: plain Python loops (math.exp) on tiny inputs.
* Against unquantized float64 attention on the bf16 inputs (relative
  Frobenius error within the few-percent E4M3 error; catches swapped scales).
* The float-input variant (BF16 baseline) against torch-CPU float64 SDPA
  directly, and against the code variant on decoded values.
* Invariants: rows of P sum to one (V = 1 gives O = 1), a one-token sequence
  returns its V row, identical keys return the mean of V, no leakage across
  cu_seqlens boundaries, key/value permutation within a sequence.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import ScaleState, attention, attention_rows, decode, quantize_qkv
from workloads import random_qkv

D = 128


def _f32(t):
    return t.float().numpy()


def _quant(seqlens, H, seed, sigma=1.0, outlier_p=0.0, outlier_scale=1.0):
    q, k, v = (_f32(t) for t in random_qkv(seqlens, H, seed, sigma=sigma, outlier_p=outlier_p,
                                           outlier_scale=outlier_scale))
    st = ScaleState()
    q8, k8, v8, descale, _ = quantize_qkv(st, "dynamic", q, k, v)
    return (q, k, v), (q8, k8, v8), descale


def _cu(seqlens):
    return np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int64)


def _sdpa64(qf, kf, vf, cu):
    out = np.zeros_like(qf)
    for b in range(len(cu) - 1):
        lo, hi = cu[b], cu[b + 1]
        if hi == lo:
            continue
        q = torch.from_numpy(np.ascontiguousarray(qf[lo:hi].transpose(1, 0, 2)))
        k = torch.from_numpy(np.ascontiguousarray(kf[lo:hi].transpose(1, 0, 2)))
        v = torch.from_numpy(np.ascontiguousarray(vf[lo:hi].transpose(1, 0, 2)))
        out[lo:hi] = torch.nn.functional.scaled_dot_product_attention(q, k, v).numpy().transpose(1, 0, 2)
    return out


def test_lossless_case_equals_torch_sdpa():
    rng = np.random.default_rng(3)
    seqlens = [5, 33, 1, 70]
    T, H = sum(seqlens), 2
    finite_codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    vals = []
    for _ in range(3):
        # every element is (E4M3 value) / 64, so |x| <= 448/64 = 7 and x * 64 is exact
        x = (decode(rng.choice(finite_codes, size=(T, H, D))) / 64.0).astype(np.float32)
        x.flat[rng.integers(x.size)] = 7.0           # amax exactly 7 -> descale 2^-6, inv 2^6
        vals.append(x)
    q, k, v = vals
    st = ScaleState()
    q8, k8, v8, descale, _ = quantize_qkv(st, "dynamic", q, k, v)
    assert np.all(descale == np.float32(2.0 ** -6))
    for x, c in zip(vals, (q8, k8, v8)):
        assert np.array_equal(decode(c) * 2.0 ** -6, x.astype(np.float64))
    cu = _cu(seqlens)
    got = attention(q8, k8, v8, descale, cu)
    ref = _sdpa64(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), cu)
    assert np.abs(got - ref).max() <= 1e-12


def test_brute_force_tiny():
    seqlens = [3, 1, 5]
    H = 2
    _, (q8, k8, v8), descale = _quant(seqlens, H, seed=11, sigma=1.5)
    got = attention(q8, k8, v8, descale, _cu(seqlens))
    qf, kf, vf = (decode(c) * float(s) for c, s in zip((q8, k8, v8), descale))
    cu = _cu(seqlens)
    for b in range(len(seqlens)):
        for h in range(H):
            for i in range(cu[b], cu[b + 1]):
                scores = []
                for j in range(cu[b], cu[b + 1]):
                    scores.append(sum(qf[i, h, d] * kf[j, h, d] for d in range(D)) / math.sqrt(D))
                mx = max(scores)
                w = [math.exp(s - mx) for s in scores]
                tot = sum(w)
                for d in range(D):
                    o = sum(w[jj] * vf[cu[b] + jj, h, d] for jj in range(len(w))) / tot
                    assert abs(got[i, h, d] - o) <= 1e-12 * max(1.0, abs(o))


def test_close_to_unquantized_attention():
    seqlens = [64, 17, 128]
    (q, k, v), (q8, k8, v8), descale = _quant(seqlens, 2, seed=21, sigma=1.0)
    # make the three tensors' ranges differ so a swapped scale would show
    got = attention(q8, k8, v8, descale, _cu(seqlens))
    ref = _sdpa64(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), _cu(seqlens))
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert rel <= 0.1, rel


def test_scales_are_not_swapped():
    rng = np.random.default_rng(5)
    seqlens = [40, 24]
    T, H = sum(seqlens), 2
    q = (rng.standard_normal((T, H, D)) * 0.05).astype(np.float32)
    k = (rng.standard_normal((T, H, D)) * 3.0).astype(np.float32)
    v = (rng.standard_normal((T, H, D)) * 40.0).astype(np.float32)
    st = ScaleState()
    q8, k8, v8, descale, _ = quantize_qkv(st, "dynamic", q, k, v)
    got = attention(q8, k8, v8, descale, _cu(seqlens))
    ref = _sdpa64(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), _cu(seqlens))
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) <= 0.1


def test_rows_sum_to_one():
    seqlens = [50, 7]
    (_, _, _), (q8, k8, _), descale = _quant(seqlens, 2, seed=31, sigma=2.0)
    ones = np.full(q8.shape, 0x38, dtype=np.uint8)      # code of 1.0
    out = attention(q8, k8, ones, np.array([descale[0], descale[1], 1.0], np.float32), _cu(seqlens))
    assert np.abs(out - 1.0).max() <= 1e-12


def test_one_token_sequence_returns_v_row():
    seqlens = [9, 1, 4]
    _, (q8, k8, v8), descale = _quant(seqlens, 2, seed=41, sigma=2.5)
    out = attention(q8, k8, v8, descale, _cu(seqlens))
    assert np.array_equal(out[9], decode(v8[9]) * float(descale[2]))


def test_identical_keys_give_mean_of_v():
    seqlens = [30]
    _, (q8, k8, v8), descale = _quant(seqlens, 2, seed=51)
    k8 = np.broadcast_to(k8[:1], k8.shape).copy()
    out = attention(q8, k8, v8, descale, _cu(seqlens))
    mean_v = (decode(v8) * float(descale[2])).mean(axis=0)
    assert np.abs(out - mean_v[None]).max() <= 1e-12


def test_no_leakage_across_sequences():
    seqlens = [20, 33, 11]
    _, (q8, k8, v8), descale = _quant(seqlens, 2, seed=61)
    cu = _cu(seqlens)
    base = attention(q8, k8, v8, descale, cu)
    k2, v2 = k8.copy(), v8.copy()
    rng = np.random.default_rng(0)
    k2[cu[1]:cu[2]] = rng.integers(0, 0x7E, size=k2[cu[1]:cu[2]].shape)
    v2[cu[1]:cu[2]] = rng.integers(0, 0x7E, size=v2[cu[1]:cu[2]].shape)
    pert = attention(q8, k2, v2, descale, cu)
    for b in (0, 2):
        assert np.array_equal(base[cu[b]:cu[b + 1]], pert[cu[b]:cu[b + 1]])
    assert not np.array_equal(base[cu[1]:cu[2]], pert[cu[1]:cu[2]])


def test_permutation_of_keys_and_values():
    seqlens = [25, 40]
    _, (q8, k8, v8), descale = _quant(seqlens, 2, seed=71)
    cu = _cu(seqlens)
    base = attention(q8, k8, v8, descale, cu)
    perm = np.arange(sum(seqlens))
    perm[cu[1]:cu[2]] = cu[1] + np.random.default_rng(1).permutation(seqlens[1])
    out = attention(q8, k8[perm], v8[perm], descale, cu)
    assert np.abs(out - base).max() <= 1e-12


def test_rows_subset_matches_full():
    seqlens = [30, 0, 45, 9]
    _, (q8, k8, v8), descale = _quant(seqlens, 2, seed=81)
    cu = _cu(seqlens)
    full = attention(q8, k8, v8, descale, cu)
    rows = np.array([0, 29, 30, 31, 74, 75, 83])
    sub = attention_rows(q8, k8, v8, descale, cu, rows)
    assert np.abs(sub - full[rows]).max() <= 1e-12


def test_cu_seqlens_validation():
    _, (q8, k8, v8), descale = _quant([8], 1, seed=91)
    for bad in ([0, 7], [1, 8], [0, 5, 3, 8], [0]):
        with pytest.raises(ValueError):
            attention(q8, k8, v8, descale, bad)


def test_magnitude_scale():
    """M = P|V|: at least |O| everywhere, equal to O when V >= 0, 1 when V = 1."""
    seqlens = [40, 9]
    _, (q8, k8, v8), descale = _quant(seqlens, 2, seed=101, sigma=2.0)
    cu = _cu(seqlens)
    out, mag = attention(q8, k8, v8, descale, cu, magnitude=True)
    assert np.array_equal(out, attention(q8, k8, v8, descale, cu))
    assert np.all(mag >= np.abs(out) - 1e-12)
    pos = v8 & 0x7F                                       # clear sign bits: V >= 0
    out_p, mag_p = attention(q8, k8, pos, descale, cu, magnitude=True)
    assert np.abs(mag_p - out_p).max() <= 1e-12
    ones = np.full(q8.shape, 0x38, dtype=np.uint8)
    _, mag_1 = attention(q8, k8, ones, np.array([descale[0], descale[1], 1.0], np.float32), cu, magnitude=True)
    assert np.abs(mag_1 - 1.0).max() <= 1e-12
    rows = np.array([0, 39, 40, 48])
    o_r, m_r = attention_rows(q8, k8, v8, descale, cu, rows, magnitude=True)
    assert np.abs(o_r - out[rows]).max() <= 1e-12 and np.abs(m_r - mag[rows]).max() <= 1e-12


def test_float_attention_equals_torch_sdpa():
    """The float-input definition (BF16 baseline) against torch-CPU float64 SDPA, per sequence."""
    rng = np.random.default_rng(31)
    seqlens = [1, 5, 0, 70, 33]
    T, H = sum(seqlens), 3
    q, k, v = (rng.standard_normal((T, H, 128)) * s for s in (2.0, 1.5, 1.0))
    cu = _cu(seqlens)
    got, mag = oracle.attention_float(q, k, v, cu, magnitude=True)
    ref = _sdpa64(q, k, v, cu)
    assert np.allclose(got, ref, rtol=0, atol=1e-12)
    assert np.all(mag >= np.abs(got) - 1e-12)
    rows = np.array([0, 3, 6, 40, 108])
    sub = oracle.attention_float_rows(q, k, v, cu, rows)
    assert np.allclose(sub, got[rows], rtol=0, atol=1e-12)


def test_float_attention_matches_code_attention_on_decoded_values():
    """attention(codes) is attention_float of the decoded, scaled codes (same definition)."""
    rng = np.random.default_rng(8)
    seqlens = [9, 40]
    T, H = sum(seqlens), 2
    codes = [rng.integers(0, 256, (T, H, 128)).astype(np.uint8) for _ in range(3)]
    for c in codes:
        c[(c & 0x7F) == 0x7F] = 0x38                      # no NaN codes
    descale = np.array([0.5, 0.25, 2.0], np.float32)
    a = oracle.attention(*codes, descale, _cu(seqlens))
    f = oracle.attention_float(*(oracle.decode(c) * float(d) for c, d in zip(codes, descale)), _cu(seqlens))
    assert np.array_equal(a, f)


def test_head_dim_80_lossless_equals_torch_sdpa():
    """Codes zero-padded to 128 dims, attention over the first 80: the scale is 1/sqrt(80) (library SDPA on the
    decoded values, which quantization reproduces exactly because every value is an E4M3 value times 2^-6)."""
    rng = np.random.default_rng(41)
    seqlens = [5, 33]
    T, H, D = sum(seqlens), 2, 80
    vals = decode(np.arange(256, dtype=np.uint8))
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= 7.0)]
    xs = []
    for _ in range(3):
        x = rng.choice(vals, size=(T, H, D)).astype(np.float64) * 2.0 ** -6
        x[0, 0, 0] = 7.0 * 2.0 ** -6             # amax exactly 7 * 2^-6: scales are powers of two
        xs.append(x)
    st = ScaleState()
    q8, k8, v8, descale, _ = quantize_qkv(st, "dynamic", *(x.astype(np.float32) for x in xs))
    got = attention(q8, k8, v8, descale, _cu(seqlens))
    ref = _sdpa64(*xs, _cu(seqlens))
    assert np.allclose(got, ref, rtol=0, atol=1e-12)
