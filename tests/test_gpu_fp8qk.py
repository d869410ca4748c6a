"""GPU: attention with Q K^T on the fp8 MFMA (qfa_fp8_varlen_attn_fp8qk) on inputs without outliers.

The entry point is for Q and K without isolated large elements (the fp8
MFMA truncates each product of a group of 8 dims below the group's largest
product).  On such inputs it is held to the same bar as qfa_fp8_varlen_attn
against the oracle:
- seeded Gaussian Q, K, V (sigma 2, no outliers) over ragged sequences that
  span several tiles, empty sequences and one-token sequences, at head dims
  128, 96 and 80 (the fp8 kernels) and 64 (the exact kernel);
- one-token sequences return their V row bit for bit;
- the largest head count the ABI accepts (65536), sequences of 2 and 1
  tokens, on sampled heads;
- the 2304-token image (static scales) on every row, and the QHD batch of
  three 14400-token images (dynamic and static scales) on sampled rows of
  each image.
"""

import numpy as np
import pytest
import torch

import oracle
import quantized_flash_attn_amd as qfa
from helpers import assert_fp8_attn_close, bf16_to_f32, codes, log, one_token_row, oracle_attention_rows
from workloads import WORKLOADS, cu_seqlens_tensor, make_qkv, random_qkv

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.mark.parametrize("D", [128, 96, 80, 64])
@pytest.mark.parametrize("seqlens", [[1], [7, 1], [255, 1, 300], [0, 513, 0, 17], [128, 129, 256, 257],
                                     [1000, 24, 389]])
def test_fp8qk_ragged(seqlens, D):
    H = 3
    log(f"fp8qk seqlens={seqlens} D={D}")
    q, k, v = random_qkv(seqlens, H, seed=300 + sum(seqlens) + D, device=DEV, sigma=2.0)
    qkv = torch.stack([q[..., :D], k[..., :D], v[..., :D]], dim=1).contiguous()
    st = qfa.init_scale_state(DEV)
    q8, k8, v8 = qfa.quantize_qkv_packed(st, "dynamic", qkv)
    descale = np.array(qfa.read_scale_state(st)["descale"], np.float32)
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    out = qfa.fp8_varlen_attn_fp8qk(q8, k8, v8, qfa.descale(st), cu_seqlens_tensor(seqlens, DEV), H, head_dim=D)
    assert tuple(out.shape) == (sum(seqlens), H, D)
    ref, mag = oracle.attention(codes(q8)[..., :D], codes(k8)[..., :D], codes(v8)[..., :D], descale, cu,
                                magnitude=True)
    assert_fp8_attn_close(bf16_to_f32(out), ref, f"fp8qk {seqlens} D={D}", mag=mag)
    for b, n in enumerate(seqlens):
        if n == 1:
            row = int(cu[b])
            want = one_token_row(codes(v8)[row, :, :D], descale[2])
            assert torch.equal(out[row].cpu().view(torch.int16), want.view(torch.int16)), row


@pytest.mark.timeout(600)
@pytest.mark.parametrize("widx,mode", [(2, "static"), (4, "dynamic"), (4, "static")])
def test_fp8qk_outlier_free_workloads(widx, mode):
    w = WORKLOADS[widx]
    assert w.outlier_p == 0.0
    log(f"fp8qk workload {widx} ({w.name}), mode {mode}")
    if mode == "static":
        sa = [oracle.amax(bf16_to_f32(t)) for t in make_qkv(w, 0, device=DEV, calibration=True)]
        st = qfa.init_scale_state(DEV, static_amax=sa, margin=1.5)
    else:
        st = qfa.init_scale_state(DEV)
    q8, k8, v8 = qfa.quantize_qkv(st, mode, *make_qkv(w, 0, device=DEV))
    descale = np.array(qfa.read_scale_state(st)["descale"], np.float32)
    out = qfa.fp8_varlen_attn_fp8qk(q8, k8, v8, qfa.descale(st), cu_seqlens_tensor(w.seqlens, DEV), w.num_heads)
    cu = np.array(w.cu_seqlens)
    if len(w.seqlens) == 1:
        rows = np.arange(w.total_tokens)
    else:   # per image: its first 256 rows, its last 256 rows and 512 seeded others
        rng = np.random.default_rng(11)
        rows = np.unique(np.concatenate([np.concatenate([np.arange(lo, lo + 256), np.arange(hi - 256, hi),
                                                         rng.integers(lo, hi, 512)])
                                         for lo, hi in zip(cu[:-1], cu[1:])]))
    log(f"  checking {rows.size} rows x {w.num_heads} heads")
    ref, mag = oracle_attention_rows(codes(q8), codes(k8), codes(v8), descale, cu, rows)
    got = bf16_to_f32(out[torch.from_numpy(rows).to(DEV)])
    assert_fp8_attn_close(got, ref, f"fp8qk workload {widx} {mode}", mag=mag)


def test_fp8qk_max_heads():
    seqlens, H = [2, 1], 65536
    log(f"fp8qk seqlens={seqlens} H={H}")
    q, k, v = random_qkv(seqlens, H, seed=47, device=DEV, sigma=1.5)
    st = qfa.init_scale_state(DEV)
    c8 = qfa.quantize_qkv(st, "dynamic", q, k, v)
    out = qfa.fp8_varlen_attn_fp8qk(*c8, qfa.descale(st), cu_seqlens_tensor(seqlens, DEV), H)
    descale = np.array(qfa.read_scale_state(st)["descale"], np.float32)
    heads = np.unique(np.concatenate([np.arange(256), np.arange(H - 256, H),
                                      np.random.default_rng(47).integers(0, H, size=512)]))
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    ref, mag = oracle.attention(*(codes(t)[:, heads] for t in c8), descale, cu, magnitude=True)
    assert_fp8_attn_close(bf16_to_f32(out)[:, heads], ref, f"fp8qk {H} heads", mag=mag)
    # the one-token sequence returns its V row
    want = one_token_row(codes(c8[2])[2, heads], descale[2])
    got = out[2, torch.from_numpy(heads).to(DEV)].cpu().view(torch.int16)
    assert torch.equal(got, want.view(torch.int16))
