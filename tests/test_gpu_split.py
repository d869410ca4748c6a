"""GPU parity of the split-key FP8 attention (qfa_fp8_varlen_attn_split) against the oracle.

Each (head, query tile)'s keys are split into ranges of whole 128-key tiles;
each range writes an fp16 partial result normalised by its own softmax sum,
plus its running max and sum, and a second kernel merges the ranges.  The
oracle is the same float64 definition as for the unsplit kernel.  Tolerance:
the contract's bound, and the E4M3 kernel's derived bound (tests/helpers.py);
the fp16 partials add at most 2^-11 M to the error, which that bound's
allowance above 2^-10 + 2^-8 covers (2^-10 + 2^-11 + 2^-8 ~= 5.4e-3 < 6e-3).
"""

import numpy as np
import pytest
import torch

import oracle
import quantized_flash_attn_amd as qfa
from helpers import (assert_fp8_attn_close, bf16_to_f32, check_rows, codes, log, one_token_row,
                     oracle_attention_rows)
from workloads import WORKLOADS, cu_seqlens_tensor, make_qkv, random_qkv

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _codes_and_oracle(q, k, v, seqlens, mode="dynamic", sa=None):
    st = qfa.init_scale_state(DEV, static_amax=sa, margin=1.5) if sa else qfa.init_scale_state(DEV)
    g = qfa.quantize_qkv(st, mode, q, k, v)
    ost = oracle.ScaleState(static_amax=sa, margin=1.5) if sa else oracle.ScaleState()
    o8q, o8k, o8v, descale, _ = oracle.quantize_qkv(ost, mode, *(bf16_to_f32(t) for t in (q, k, v)))
    for gg, oo in zip(g, (o8q, o8k, o8v)):
        assert np.array_equal(codes(gg), oo)
    return st, g, (o8q, o8k, o8v), descale


@pytest.mark.parametrize("seqlens,H,splits", [
    ([1000, 24, 389], 3, 2),
    ([1000, 24, 389], 3, 3),
    ([1000, 24, 389], 3, 5),
    ([1000, 24, 389], 3, 16),      # more ranges than key tiles: most ranges are empty
    ([0, 513, 0, 17], 2, 4),       # empty sequences
    ([1], 2, 16),                  # one key: fifteen empty ranges
    ([256, 257, 384], 2, 3),       # query and key tile boundaries
    ([2304], 4, 0),                # the automatic count (7 ranges)
])
def test_split_matches_oracle(seqlens, H, splits):
    log(f"split seqlens={seqlens} H={H} splits={splits}")
    q, k, v = random_qkv(seqlens, H, seed=sum(seqlens) * 3 + H + splits, device=DEV, sigma=2.0, outlier_p=0.001,
                         outlier_scale=20.0)
    st, (q8, k8, v8), oc, descale = _codes_and_oracle(q, k, v, seqlens)
    cu = cu_seqlens_tensor(seqlens, DEV)
    out = qfa.fp8_varlen_attn_split(q8, k8, v8, qfa.descale(st), cu, H, num_splits=splits)
    ref, mag = oracle.attention(*oc, descale, np.concatenate([[0], np.cumsum(seqlens)]), magnitude=True)
    assert_fp8_attn_close(bf16_to_f32(out), ref, f"split {splits} seqlens {seqlens}", mag=mag)


def test_one_split_is_the_unsplit_kernel():
    seqlens, H = [700, 33, 129], 2
    q, k, v = random_qkv(seqlens, H, seed=77, device=DEV, sigma=1.5)
    st, (q8, k8, v8), _, _ = _codes_and_oracle(q, k, v, seqlens)
    cu = cu_seqlens_tensor(seqlens, DEV)
    a = qfa.fp8_varlen_attn(q8, k8, v8, qfa.descale(st), cu, H)
    b = qfa.fp8_varlen_attn_split(q8, k8, v8, qfa.descale(st), cu, H, num_splits=1,
                                  workspace=torch.empty(0, dtype=torch.uint8, device=DEV))
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_split_one_token_rows_and_determinism():
    """A one-key row is its value row bit for bit through the merge too (weight 2^4 exactly), and repeated
    split launches give the same bits."""
    seqlens, H = [5, 1, 300, 1], 2
    q, k, v = random_qkv(seqlens, H, seed=13, device=DEV, sigma=2.0)
    st, (q8, k8, v8), _, _ = _codes_and_oracle(q, k, v, seqlens)
    cu = cu_seqlens_tensor(seqlens, DEV)
    out1 = qfa.fp8_varlen_attn_split(q8, k8, v8, qfa.descale(st), cu, H, num_splits=4)
    out2 = qfa.fp8_varlen_attn_split(q8, k8, v8, qfa.descale(st), cu, H, num_splits=4)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    s_v = np.float32(qfa.read_scale_state(st)["descale"][2])
    for row in (5, 306):
        want = one_token_row(codes(v8)[row], s_v)
        assert torch.equal(out1[row].cpu().view(torch.int16), want.view(torch.int16)), row


def test_split_no_leakage():
    seqlens, H = [300, 129, 640, 500], 2
    q, k, v = random_qkv(seqlens, H, seed=19, device=DEV)
    st = qfa.init_scale_state(DEV, static_amax=[8.0, 8.0, 8.0], margin=1.0)
    q8, k8, v8 = qfa.quantize_qkv(st, "static", q, k, v)
    cu_t = cu_seqlens_tensor(seqlens, DEV)
    out1 = qfa.fp8_varlen_attn_split(q8, k8, v8, qfa.descale(st), cu_t, H, num_splits=3)
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    k2, v2 = k.clone(), v.clone()
    k2[cu[1]:cu[2]] = torch.randn_like(k2[cu[1]:cu[2]].float()).to(torch.bfloat16) * 5
    v2[cu[1]:cu[2]] = torch.randn_like(v2[cu[1]:cu[2]].float()).to(torch.bfloat16) * 5
    q8b, k8b, v8b = qfa.quantize_qkv(st, "static", q, k2, v2)
    out2 = qfa.fp8_varlen_attn_split(q8b, k8b, v8b, qfa.descale(st), cu_t, H, num_splits=3)
    for b in (0, 2, 3):
        assert torch.equal(out1[cu[b]:cu[b + 1]].view(torch.int16), out2[cu[b]:cu[b + 1]].view(torch.int16)), b
    assert not torch.equal(out1[cu[1]:cu[2]], out2[cu[1]:cu[2]])


@pytest.mark.parametrize("D", [80, 72])
def test_split_padded_head_dim(D):
    seqlens, H = [1024, 2304, 17], 4
    q, k, v = random_qkv(seqlens, H, seed=D, device=DEV, sigma=2.0, outlier_p=0.001, outlier_scale=20.0)
    qkv = torch.stack([q[..., :D], k[..., :D], v[..., :D]], dim=1).contiguous()
    st = qfa.init_scale_state(DEV)
    q8, k8, v8 = qfa.quantize_qkv_packed(st, "dynamic", qkv)
    oq, ok, ov, descale, _ = oracle.quantize_qkv_packed(oracle.ScaleState(), "dynamic", bf16_to_f32(qkv))
    out = qfa.fp8_varlen_attn_split(q8, k8, v8, qfa.descale(st), cu_seqlens_tensor(seqlens, DEV), H, head_dim=D,
                                    num_splits=5)
    assert tuple(out.shape) == (sum(seqlens), H, D)
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    ref, mag = oracle.attention(oq[..., :D], ok[..., :D], ov[..., :D], descale, cu, magnitude=True)
    assert_fp8_attn_close(bf16_to_f32(out), ref, f"split D={D}", mag=mag)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("widx,splits", [(1, 2), (2, 3), (2, 16)])
def test_split_small_workloads(widx, splits):
    """The small images at full size split into key ranges, last forward, every row."""
    w = WORKLOADS[widx]
    mode = w.modes[0]
    log(f"split workload {widx} ({w.name}), mode {mode}, {splits} ranges")
    sa = None
    if mode == "static":
        sa = [oracle.amax(bf16_to_f32(t)) for t in make_qkv(w, 0, device=DEV, calibration=True)]
    st = qfa.init_scale_state(DEV, static_amax=sa, margin=1.5) if sa else qfa.init_scale_state(DEV)
    ost = oracle.ScaleState(static_amax=sa, margin=1.5) if sa else oracle.ScaleState()
    for fwd in range(w.forwards):
        xs = make_qkv(w, fwd, device=DEV)
        g = qfa.quantize_qkv(st, mode, *xs)
        o = oracle.quantize_qkv(ost, mode, *(bf16_to_f32(t) for t in xs))
        for gg, oo in zip(g, o[:3]):
            assert np.array_equal(codes(gg), oo), fwd
    cu = cu_seqlens_tensor(w.seqlens, DEV)
    out = qfa.fp8_varlen_attn_split(*g, qfa.descale(st), cu, w.num_heads, num_splits=splits)
    rows = check_rows(w)
    ref, mag = oracle_attention_rows(*o[:3], o[3], np.array(w.cu_seqlens), rows)
    assert_fp8_attn_close(bf16_to_f32(out)[rows], ref, f"split workload {widx} ({splits} ranges)", mag=mag)
