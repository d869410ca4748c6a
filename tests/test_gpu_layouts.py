"""GPU: both register layouts of the E4M3 attention on the same edge cases.

The library runs the 32x32 layout for launches of at most 3/4 as many
workgroups as the device has CUs, and the 16x16 layout for larger ones (head
dims above 96).  Each case here runs twice on the same per-head data: with 2
heads (a few workgroups: the 32x32 layout) and with 512 heads, whose first two
are those same heads (more workgroups than any device has CUs: the 16x16
layout).  Both outputs of the first two heads must meet the contract against
the oracle, the 512-head run also on sampled other heads, and a one-token
sequence must return its V row bit for bit in both.
"""

import numpy as np
import pytest
import torch

import oracle
import quantized_flash_attn_amd as qfa
from helpers import assert_fp8_attn_close, bf16_to_f32, codes, log, one_token_row
from workloads import cu_seqlens_tensor, random_qkv

pytestmark = pytest.mark.gpu

DEV = "cuda"
H_BIG = 512


def _run(q, k, v, seqlens, H):
    st = qfa.init_scale_state(DEV, static_amax=[40.0, 40.0, 40.0], margin=1.0)
    q8, k8, v8 = qfa.quantize_qkv(st, "static", q[:, :H].contiguous(), k[:, :H].contiguous(), v[:, :H].contiguous())
    out = qfa.fp8_varlen_attn(q8, k8, v8, qfa.descale(st), cu_seqlens_tensor(seqlens, DEV), H)
    return (q8, k8, v8), out, qfa.read_scale_state(st)["descale"]


@pytest.mark.parametrize("seqlens", [[1], [7, 1], [255, 1, 300], [0, 513, 0, 17], [128, 129, 256, 257]])
def test_layouts_agree_with_the_oracle(seqlens):
    log(f"layouts seqlens={seqlens}")
    q, k, v = random_qkv(seqlens, H_BIG, seed=71 + sum(seqlens), device=DEV, sigma=2.0, outlier_p=0.001,
                         outlier_scale=20.0)
    (q8s, k8s, v8s), small, ds = _run(q, k, v, seqlens, 2)
    (q8b, k8b, v8b), big, db = _run(q, k, v, seqlens, H_BIG)
    # static scales: the two heads' codes are the same in both runs
    assert ds == db
    assert torch.equal(q8s, q8b[:, :2]) and torch.equal(k8s, k8b[:, :2]) and torch.equal(v8s, v8b[:, :2])
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    descale = np.array(ds, np.float32)
    heads = [0, 1, 97, 300, H_BIG - 1]
    ref, mag = oracle.attention(codes(q8b)[:, heads], codes(k8b)[:, heads], codes(v8b)[:, heads], descale, cu,
                                magnitude=True)
    assert_fp8_attn_close(bf16_to_f32(small), ref[:, :2], f"{seqlens}, 2 heads (32x32)", mag=mag[:, :2])
    assert_fp8_attn_close(bf16_to_f32(big)[:, heads], ref, f"{seqlens}, {H_BIG} heads (16x16)", mag=mag)
    # one-token sequences: the value row, bit for bit, in both layouts
    for b, n in enumerate(seqlens):
        if n != 1:
            continue
        row = int(cu[b])
        for out, v8, h in ((small, v8s, 0), (small, v8s, 1), (big, v8b, 0), (big, v8b, H_BIG - 1)):
            want = one_token_row(codes(v8)[row, h], ds[2])
            assert torch.equal(out[row, h].cpu().view(torch.int16), want.view(torch.int16)), (row, h)
