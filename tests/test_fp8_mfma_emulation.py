"""What the fp8 MFMAs' summation does to the workloads' attention (CPU).

The exact E4M3 attention kernel runs Q K^T on the fp16 MFMA over exactly
converted codes, at half the fp8 rate; qfa_fp8_varlen_attn_fp8qk runs it on
v_mfma_f32_16x16x128_f8f6f4 for inputs without outliers
(tests/test_gpu_fp8qk.py checks it on the GPU).
tests/test_gpu_mfma_hw.py pins how gfx950's fp8 MFMAs sum: within each group
of 8 consecutive products, every product is cut toward zero to a multiple of
2^(E - 13), E the exponent of the group's largest product; the groups and
the accumulator are then added exactly.  This test emulates that summation
in float64 (pinned to the probe's observed values), computes attention with
it on the workloads' own codes, and compares with the exact logits, under the
contract's measure e = |g - r| / max(1, |r|):

* the two outlier-free workloads stay far inside the contract, even on the
  query rows with the largest codes: the 2304-token image (workload 2,
  N(0, sigma_h) Q and K, static scales) and one 14400-token image of the QHD
  batch (workload 4, the same distribution, dynamic scales);
* the kernel-benchmark workload (workload 3: x20 outliers in 0.1 % of Q and K
  elements) breaks it on the rows that hold outliers: a product of two
  outliers truncates its 7 group-mates and moves the row's dominant logits.

* on seeded Gaussian inputs the error grows with the logits' scale
  (sigma^2) times the outliers' size: sigma 1 keeps x20 outliers (0.1 % of
  the elements) inside the contract, sigma 3 does not keep x10 ones.

So fp8 Q K^T is exact enough only for inputs known to be free of outliers,
which the per-tensor scales cannot tell apart, and not for the workload the
library is measured on: that is the domain of the fp8 entry point, and the
default path stays on the fp16 MFMA.
"""

import numpy as np
import pytest

import oracle
from test_gpu_mfma_hw import CASES, FP8_OBSERVED
from workloads import WORKLOADS, make_qkv, random_qkv

TOL_MAX = 3e-2


def fp8_mfma_logits(q, k):
    """Q K^T with gfx950's fp8-MFMA group summation.  q [r, 128], k [n, 128]
    (E4M3 values, float64) -> [r, n]."""
    prod = q[:, None, :] * k[None, :, :]
    groups = prod.reshape(prod.shape[0], prod.shape[1], -1, 8)
    top = np.abs(groups).max(-1, keepdims=True)
    quantum = 2.0 ** (np.floor(np.log2(np.where(top > 0, top, 1.0))) - 13)
    return (np.trunc(groups / quantum) * quantum).sum((-1, -2))


def test_emulation_matches_the_probe():
    for (name, a, b, c00, exact), want in zip(CASES, FP8_OBSERVED["f8f6f4_k128"]):
        qa = np.zeros((1, 128))
        kb = np.zeros((1, 128))
        qa[0, :len(a)] = a
        kb[0, :len(b)] = b
        got = c00 + fp8_mfma_logits(qa, kb)[0, 0]
        assert got == want, (name, got, want)
        assert float((qa * kb).sum() + c00) == exact, name


def _codes(widx, mode, num_tokens=None):
    w = WORKLOADS[widx]
    if mode == "static":
        sa = [oracle.amax(t.float().numpy()) for t in make_qkv(w, 0, calibration=True, num_tokens=num_tokens)]
        st = oracle.ScaleState(static_amax=sa, margin=1.5)
    else:
        st = oracle.ScaleState()
    x = (t.float().numpy() for t in make_qkv(w, 0, num_tokens=num_tokens))
    q8, k8, v8, descale, _ = oracle.quantize_qkv(st, mode, *x)
    return w, q8, k8, v8, descale


def _fp8_mfma_logits_chunked(q, k, keys=1024):
    return np.concatenate([fp8_mfma_logits(q, k[j:j + keys]) for j in range(0, k.shape[0], keys)], axis=1)


def _worst_error(widx, mode, heads, rows_per_head, num_tokens=None):
    """Max contract error over the given heads' rows_per_head query rows with
    the largest |code| (the rows holding outliers), first sequence.  With
    num_tokens, the tokens drawn are only that many (the first sequence's
    length), and the codes and scales come from them alone."""
    w, q8, k8, v8, (s_q, s_k, s_v) = _codes(widx, mode, num_tokens)
    lo, hi = w.cu_seqlens[0], w.cu_seqlens[1]
    assert hi <= q8.shape[0]
    c = float(s_q) * float(s_k) / np.sqrt(128.0)
    worst = 0.0
    for h in heads:
        q = oracle.decode(q8[lo:hi, h]).astype(np.float64)
        k = oracle.decode(k8[lo:hi, h]).astype(np.float64)
        v = oracle.decode(v8[lo:hi, h]).astype(np.float64) * float(s_v)
        rows = np.argsort(-np.abs(q).max(-1), kind="stable")[:rows_per_head]

        def attend(s):
            z = s * c
            p = np.exp(z - z.max(-1, keepdims=True))
            return (p / p.sum(-1, keepdims=True)) @ v

        r = attend(q[rows] @ k.T)
        if h == heads[0]:   # the exact side is the oracle's attention on the same codes
            ref = oracle.attention_rows(q8[:, h:h + 1], k8[:, h:h + 1], v8[:, h:h + 1], (s_q, s_k, s_v),
                                        np.array([lo, hi]), lo + rows)
            assert np.allclose(r, ref[:, 0], rtol=1e-12, atol=1e-12)
        g = attend(_fp8_mfma_logits_chunked(q[rows], k))
        worst = max(worst, float((np.abs(g - r) / np.maximum(1.0, np.abs(r))).max()))
    print(f"workload {widx} ({mode}): fp8-MFMA Q K^T, max e {worst:.3e}", flush=True)
    return worst


def test_outlier_free_image_stays_inside_the_contract():
    assert _worst_error(2, "static", range(16), 64) < 0.1 * TOL_MAX


@pytest.mark.timeout(300)
def test_outlier_free_qhd_image_stays_inside_the_contract():
    # one 14400-token image of the QHD batch: per-head sigma Q and K, unit V
    assert _worst_error(4, "dynamic", (0, 5, 11, 15), 32, num_tokens=WORKLOADS[4].seqlens[0]) < 0.1 * TOL_MAX


@pytest.mark.timeout(300)
def test_outliers_break_the_contract():
    # heads 1 and 4 of the first forward: among their 128 query rows with the
    # largest codes are rows whose leading logits the truncation moves far
    # enough to shift the softmax weights
    assert _worst_error(3, "dynamic", (1, 4), 128) > TOL_MAX


def _random_case_error(sigma, scale, T=2048, H=4, seed=23, rows_per_head=48):
    """Max contract error of fp8-MFMA Q K^T on Gaussian Q, K, V of standard deviation sigma with 0.1 % of the
    elements `scale` times larger (dynamic scales), over each head's rows with the largest |code|."""
    q, k, v = random_qkv([T], H, seed=seed, sigma=sigma, outlier_p=0.001, outlier_scale=scale)
    q8, k8, v8, (s_q, s_k, s_v), _ = oracle.quantize_qkv(oracle.ScaleState(), "dynamic",
                                                         *(t.float().numpy() for t in (q, k, v)))
    c = float(s_q) * float(s_k) / np.sqrt(128.0)
    worst = 0.0
    for h in range(H):
        qd = oracle.decode(q8[:, h]).astype(np.float64)
        kd = oracle.decode(k8[:, h]).astype(np.float64)
        vd = oracle.decode(v8[:, h]).astype(np.float64) * float(s_v)
        rows = np.argsort(-np.abs(qd).max(-1), kind="stable")[:rows_per_head]

        def attend(s):
            z = s * c
            p = np.exp(z - z.max(-1, keepdims=True))
            return (p / p.sum(-1, keepdims=True)) @ vd

        r = attend(qd[rows] @ kd.T)
        g = attend(_fp8_mfma_logits_chunked(qd[rows], kd))
        worst = max(worst, float((np.abs(g - r) / np.maximum(1.0, np.abs(r))).max()))
    return worst


@pytest.mark.timeout(300)
def test_domain_depends_on_logit_scale_and_outlier_size():
    # the error grows with the logits' scale (sigma^2) times the outliers' size: unit-sigma inputs keep x20
    # outliers inside the contract, sigma-3 inputs do not keep x10 ones
    assert _random_case_error(1.0, 20.0) < TOL_MAX
    assert _random_case_error(3.0, 10.0) > TOL_MAX
