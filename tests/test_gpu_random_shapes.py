"""GPU: seeded random shapes through the whole path, against the oracle.

Each case draws, from numpy's PCG64 seeded with 1000 + case:
- 1 to 8 sequences, each with probability 0.25 an edge length from
  {0, 1, 127, 128, 129, 255, 256, 257} (empty sequences, single keys, tile
  boundaries), else a length uniform in [1, 600];
- 1 to 4 heads;
- head_dim 128 with probability 0.5, else a multiple of 8 in [8, 120];
- sigma uniform in [0.5, 3], with x20 outliers in 0.1 % of the elements or none;
- 2 to 6 key ranges for the split launch.

The path is the fused-QKV quantize (dynamic, from [T, 3, H, D]) and both
attention launches: unsplit, and split into the drawn number of ranges.
Cases drawn without outliers also run the attention with Q K^T on the fp8
MFMA (qfa_fp8_varlen_attn_fp8qk, whose domain they are), to the same bar.
Codes and scales must match the oracle bit for bit; both outputs are held to
the contract's tolerance and the kernel's own bound (tests/helpers.py)
against the oracle's float64 attention over the D real dims.  Every case
stays under 2000 tokens, so the oracle checks every output row.
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
EDGE_LENGTHS = (0, 1, 127, 128, 129, 255, 256, 257)


def draw_case(i):
    rng = np.random.default_rng(1000 + i)
    n = int(rng.integers(1, 9))
    seqlens = [int(rng.choice(EDGE_LENGTHS)) if rng.random() < 0.25 else int(rng.integers(1, 601)) for _ in range(n)]
    if sum(seqlens) == 0:
        seqlens[0] = 1
    while sum(seqlens) > 2000:
        seqlens.pop()
    H = int(rng.integers(1, 5))
    D = 128 if rng.random() < 0.5 else 8 * int(rng.integers(1, 16))
    sigma = float(rng.uniform(0.5, 3.0))
    outliers = 0.001 if rng.random() < 0.5 else 0.0
    splits = int(rng.integers(2, 7))
    return seqlens, H, D, sigma, outliers, splits


@pytest.mark.parametrize("case", range(24))
def test_random_shape(case):
    seqlens, H, D, sigma, outliers, splits = draw_case(case)
    log(f"case {case}: seqlens={seqlens} H={H} D={D} sigma={sigma:.2f} outliers={outliers} splits={splits}")
    q, k, v = random_qkv(seqlens, H, seed=5000 + case, device=DEV, sigma=sigma, outlier_p=outliers,
                         outlier_scale=20.0)
    qkv = torch.stack([q[..., :D], k[..., :D], v[..., :D]], dim=1).contiguous()

    st = qfa.init_scale_state(DEV)
    q8, k8, v8 = qfa.quantize_qkv_packed(st, "dynamic", qkv)
    oq, ok, ov, descale, _ = oracle.quantize_qkv_packed(oracle.ScaleState(), "dynamic", bf16_to_f32(qkv))
    for g, o in zip((q8, k8, v8), (oq, ok, ov)):
        assert np.array_equal(codes(g), o)
    assert np.array_equal(np.array(qfa.read_scale_state(st)["descale"], np.float32), descale)

    cu = cu_seqlens_tensor(seqlens, DEV)
    ref, mag = oracle.attention(oq[..., :D], ok[..., :D], ov[..., :D], descale,
                                np.concatenate([[0], np.cumsum(seqlens)]), magnitude=True)
    out = qfa.fp8_varlen_attn(q8, k8, v8, qfa.descale(st), cu, H, head_dim=D)
    assert tuple(out.shape) == (sum(seqlens), H, D)
    assert_fp8_attn_close(bf16_to_f32(out), ref, f"case {case} unsplit", mag=mag)
    out_s = qfa.fp8_varlen_attn_split(q8, k8, v8, qfa.descale(st), cu, H, head_dim=D, num_splits=splits)
    assert_fp8_attn_close(bf16_to_f32(out_s), ref, f"case {case} split {splits}", mag=mag)
    if outliers == 0.0:
        out_f = qfa.fp8_varlen_attn_fp8qk(q8, k8, v8, qfa.descale(st), cu, H, head_dim=D)
        assert_fp8_attn_close(bf16_to_f32(out_f), ref, f"case {case} fp8 Q K^T", mag=mag)
