"""GPU: quantize straight from a fused QKV projection output, head dims below 128, FP8 attention on padded codes.

"FP8 ViT Encoder Attention" (Performance) counts the split into three
quantization launches and the head-dim un-padding among the overheads that
make small images slow.  The packed path reads [T, 3, H, D] once, writes codes
[T, H, 128] zero-padded past D, and the attention kernel reads those and
writes [T, H, D].  Codes and scales are compared bit-exactly with the oracle
(quantize_qkv_packed); attention within the tolerances of tests/helpers.py,
against the oracle's float64 attention over the D real dims (scale 1/sqrt(D)).
"""

import numpy as np
import pytest
import torch

import oracle
import quantized_flash_attn_amd as qfa
from helpers import assert_fp8_attn_close, bf16_to_f32, codes, log
from workloads import cu_seqlens_tensor, random_qkv

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _packed(seqlens, H, D, seed, sigma=1.0, outlier_p=0.0):
    """bf16 [T, 3, H, D] built from three seeded draws (Q, K, V)."""
    q, k, v = random_qkv(seqlens, H, seed=seed, device=DEV, sigma=sigma, outlier_p=outlier_p, outlier_scale=20.0)
    return torch.stack([q[..., :D], k[..., :D], v[..., :D]], dim=1).contiguous()


@pytest.mark.parametrize("D", [8, 64, 72, 80, 96, 128])
def test_packed_quantize_bit_exact(D):
    seqlens, H = [300, 77], 3
    st = qfa.init_scale_state(DEV)
    ost = oracle.ScaleState()
    for fwd in range(3):
        qkv = _packed(seqlens, H, D, seed=100 * D + fwd, sigma=1.0 + fwd, outlier_p=0.002)
        g = qfa.quantize_qkv_packed(st, "dynamic", qkv)
        o8q, o8k, o8v, descale, _ = oracle.quantize_qkv_packed(ost, "dynamic", bf16_to_f32(qkv))
        for gg, oo in zip(g, (o8q, o8k, o8v)):
            assert np.array_equal(codes(gg), oo), (D, fwd)
        snap = qfa.read_scale_state(st)
        assert np.array_equal(np.array(snap["descale"], np.float32), descale)
        assert snap["cursor"] == fwd + 1
    # static mode on the same state type
    sa = [3.0, 40.0, 0.5]
    st = qfa.init_scale_state(DEV, static_amax=sa, margin=1.5)
    qkv = _packed(seqlens, H, D, seed=7 * D, sigma=2.0)
    g = qfa.quantize_qkv_packed(st, "static", qkv)
    o = oracle.quantize_qkv_packed(oracle.ScaleState(static_amax=sa, margin=1.5), "static", bf16_to_f32(qkv))
    for gg, oo in zip(g, o[:3]):
        assert np.array_equal(codes(gg), oo), D


def test_packed_128_equals_separate_path():
    seqlens, H = [513, 1, 200], 4
    qkv = _packed(seqlens, H, 128, seed=5, sigma=2.0, outlier_p=0.001)
    a = qfa.quantize_qkv_packed(qfa.init_scale_state(DEV), "dynamic", qkv)
    sb = qfa.init_scale_state(DEV)
    b = qfa.quantize_qkv(sb, "dynamic", *(qkv[:, i].contiguous() for i in range(3)))
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    cu = cu_seqlens_tensor(seqlens, DEV)
    out_a = qfa.fp8_varlen_attn(*a, qfa.descale(sb), cu, H)
    out_b = qfa.fp8_varlen_attn(*b, qfa.descale(sb), cu, H, head_dim=128)
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))


@pytest.mark.parametrize("seqlens,H,D", [
    ([1], 2, 80),
    ([129, 7], 3, 72),
    ([300, 0, 257], 2, 80),
    ([1000, 24], 2, 64),
    ([400, 33], 2, 8),
    ([1024, 2304, 17], 16, 80),      # ViT-style: 16 heads of 80 dims
])
def test_padded_attention(seqlens, H, D):
    log(f"padded attention seqlens={seqlens} H={H} D={D}")
    qkv = _packed(seqlens, H, D, seed=sum(seqlens) + D, sigma=2.0, outlier_p=0.001)
    st = qfa.init_scale_state(DEV)
    q8, k8, v8 = qfa.quantize_qkv_packed(st, "dynamic", qkv)
    out = qfa.fp8_varlen_attn(q8, k8, v8, qfa.descale(st), cu_seqlens_tensor(seqlens, DEV), H, head_dim=D)
    assert tuple(out.shape) == (sum(seqlens), H, D)
    oq, ok, ov, descale, _ = oracle.quantize_qkv_packed(oracle.ScaleState(), "dynamic", bf16_to_f32(qkv))
    for gg, oo in zip((q8, k8, v8), (oq, ok, ov)):
        assert np.array_equal(codes(gg), oo)
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    ref, mag = oracle.attention(oq[..., :D], ok[..., :D], ov[..., :D], descale, cu, magnitude=True)
    assert_fp8_attn_close(bf16_to_f32(out), ref, f"D={D} seqlens {seqlens}", mag=mag)
