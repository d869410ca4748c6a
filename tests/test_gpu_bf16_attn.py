"""GPU parity of the BF16 varlen attention (the baseline of the FP8 path) against the oracle.

The kernel runs through the C ABI on bf16 Q, K, V; the oracle evaluates the
plain float64 definition on host copies of the same bf16 values
(``oracle.attention_float``).  Tolerance: the contract's bound, and
``TOL_MAX_BF16`` / ``TOL_MEAN_BF16`` on the P|V|-normalised error, derived in
tests/helpers.py from the kernel's arithmetic.
"""

import numpy as np
import pytest
import torch

import oracle
import quantized_flash_attn_amd as qfa
from helpers import (TOL_MAX_BF16, TOL_MEAN_BF16, assert_attn_close, bf16_to_f32, check_rows, log,
                     oracle_attention_rows)
from workloads import WORKLOADS, cu_seqlens_tensor, make_qkv, ramp_qkv, random_qkv

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _close(got, ref, what, mag):
    """The contract's bound on |r|, and the kernel's derived bound on P|V|."""
    assert_attn_close(got, ref, what, mag=mag, derived=(TOL_MAX_BF16, TOL_MEAN_BF16))


@pytest.mark.parametrize("seqlens,H,sigma,outliers", [
    ([1], 1, 1.0, 0.0),
    ([7], 2, 1.0, 0.0),
    ([128], 2, 2.0, 0.0),
    ([129], 3, 1.0, 0.001),
    ([255, 1, 300], 2, 3.0, 0.001),
    ([0, 513, 0, 17], 2, 1.5, 0.0),
    ([1000, 24, 389], 3, 2.5, 0.002),
    ([2, 3, 5, 7, 11, 13, 17, 19, 23, 29, 31, 37, 41, 43, 47, 53], 1, 1.0, 0.0),
    ([256, 257, 384], 2, 1.0, 0.001),
])
def test_small_ragged(seqlens, H, sigma, outliers):
    log(f"bf16 seqlens={seqlens} H={H} sigma={sigma}")
    q, k, v = random_qkv(seqlens, H, seed=sum(seqlens) * 11 + H, device=DEV, sigma=sigma, outlier_p=outliers,
                         outlier_scale=20.0)
    out = qfa.bf16_varlen_attn(q, k, v, cu_seqlens_tensor(seqlens, DEV), H)
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    ref, mag = oracle.attention_float(*(bf16_to_f32(t) for t in (q, k, v)), cu, magnitude=True)
    _close(bf16_to_f32(out), ref, f"seqlens {seqlens}", mag)


@pytest.mark.parametrize("order", ["increasing", "decreasing"])
def test_running_max_moves(order):
    """Logits rising along the keys rescale O and l at every key tile; falling ones never after the first."""
    seqlens = [1000, 333, 129]
    log(f"bf16 {order} logits, seqlens={seqlens}")
    q, k, v = ramp_qkv(seqlens, 2, seed=31, device=DEV, order=order)
    out = qfa.bf16_varlen_attn(q, k, v, cu_seqlens_tensor(seqlens, DEV), 2)
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    ref, mag = oracle.attention_float(*(bf16_to_f32(t) for t in (q, k, v)), cu, magnitude=True)
    _close(bf16_to_f32(out), ref, f"{order} logits", mag)


def test_one_token_sequence_returns_v_row():
    """A one-key softmax is exactly 1: the output row is the V row (p = 2^8 exactly in bf16)."""
    seqlens = [5, 1, 9, 1]
    q, k, v = random_qkv(seqlens, 2, seed=23, device=DEV, sigma=2.0)
    out = qfa.bf16_varlen_attn(q, k, v, cu_seqlens_tensor(seqlens, DEV), 2)
    for row in (5, 15):
        assert torch.equal(out[row].view(torch.int16), v[row].view(torch.int16)), row


def test_identical_keys_give_mean_of_v():
    seqlens = [300]
    q, k, v = random_qkv(seqlens, 2, seed=29, device=DEV)
    k = k[:1].expand_as(k).contiguous()
    out = qfa.bf16_varlen_attn(q, k, v, cu_seqlens_tensor(seqlens, DEV), 2)
    vh = bf16_to_f32(v).astype(np.float64)
    _close(bf16_to_f32(out), np.broadcast_to(vh.mean(axis=0), out.shape), "identical keys",
           np.broadcast_to(np.abs(vh).mean(axis=0), out.shape))


def test_no_leakage_and_determinism():
    seqlens = [300, 129, 64, 500]
    q, k, v = random_qkv(seqlens, 2, seed=31, device=DEV)
    cu_t = cu_seqlens_tensor(seqlens, DEV)
    out1 = qfa.bf16_varlen_attn(q, k, v, cu_t, 2)
    out2 = qfa.bf16_varlen_attn(q, k, v, cu_t, 2)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16)), "not deterministic"
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    k2, v2 = k.clone(), v.clone()
    k2[cu[1]:cu[2]] = torch.randn_like(k2[cu[1]:cu[2]].float()).to(torch.bfloat16) * 5
    v2[cu[1]:cu[2]] = torch.randn_like(v2[cu[1]:cu[2]].float()).to(torch.bfloat16) * 5
    out3 = qfa.bf16_varlen_attn(q, k2, v2, cu_t, 2)
    for b in (0, 2, 3):
        assert torch.equal(out1[cu[b]:cu[b + 1]].view(torch.int16), out3[cu[b]:cu[b + 1]].view(torch.int16)), b
    assert not torch.equal(out1[cu[1]:cu[2]], out3[cu[1]:cu[2]])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("widx", [1, 2, 3, 4, 5])
def test_workload_attention(widx):
    """Full-size workloads (the last forward's draws), every stated row vs the oracle."""
    w = WORKLOADS[widx]
    log(f"bf16 workload {widx} ({w.name})")
    q, k, v = make_qkv(w, w.forwards - 1, device=DEV)
    out = qfa.bf16_varlen_attn(q, k, v, cu_seqlens_tensor(w.seqlens, DEV), w.num_heads)
    torch.cuda.synchronize()
    rows = check_rows(w)
    cu = np.array(w.cu_seqlens)
    seqs = np.unique(np.searchsorted(cu, rows, side="right") - 1)
    log(f"  checking {rows.size} rows x {w.num_heads} heads in sequences {seqs.tolist()}")
    rows_t = torch.from_numpy(rows).to(DEV)
    qh = np.zeros((w.total_tokens, w.num_heads, 128), np.float32)
    kh, vh = np.zeros_like(qh), np.zeros_like(qh)
    qh[rows] = bf16_to_f32(q[rows_t])
    for b in seqs:
        lo, hi = cu[b], cu[b + 1]
        kh[lo:hi] = bf16_to_f32(k[lo:hi])
        vh[lo:hi] = bf16_to_f32(v[lo:hi])
    ref, mag = oracle_attention_rows(qh, kh, vh, None, cu, rows, codes=False)
    _close(bf16_to_f32(out[rows_t]), ref, f"bf16 workload {widx}", mag)
