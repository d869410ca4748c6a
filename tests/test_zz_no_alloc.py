"""GPU: the no-allocation split attention entry point against the workspace one.

qfa_fp8_varlen_attn_split_noalloc runs the kernels of
qfa_fp8_varlen_attn_split on the library's own fixed device array instead of
a caller-owned workspace, so on the same inputs and split count the two must
give the same bits.  Two calls in a row, the second on a smaller input,
check that the array's leftover contents from a call do not leak into the
next.  The result is also checked against the oracle (the contract's bound
and the kernel's derived bound, tests/helpers.py).
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import quantized_flash_attn_amd as qfa
from helpers import assert_fp8_attn_close, bf16_to_f32, codes, log
from workloads import cu_seqlens_tensor, random_qkv

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _call_noalloc(q8, k8, v8, scales, cu, B, T, H, splits, out):
    lib = qfa.raw_library()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.qfa_fp8_varlen_attn_split_noalloc(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), scales.data_ptr(),
                                                 cu.data_ptr(), B, T, H, 128, splits, out.data_ptr(), stream)


def test_noalloc_matches_workspace_entry_on_two_calls():
    cases = [([2304], 8, 0, 101),           # the automatic count: 3 ranges over 72 query tiles
             ([1000, 24, 389], 3, 5, 102)]  # a smaller input next, 5 ranges
    for seqlens, H, splits, seed in cases:
        T, B = sum(seqlens), len(seqlens)
        log(f"no-alloc call: seqlens={seqlens} H={H} splits={splits}")
        q, k, v = random_qkv(seqlens, H, seed=seed, device=DEV, sigma=2.0, outlier_p=0.001, outlier_scale=20.0)
        st = qfa.init_scale_state(DEV)
        q8, k8, v8 = qfa.quantize_qkv(st, "dynamic", q, k, v)
        o8 = oracle.quantize_qkv(oracle.ScaleState(), "dynamic", *(bf16_to_f32(t) for t in (q, k, v)))
        for gg, oo in zip((q8, k8, v8), o8[:3]):
            assert np.array_equal(codes(gg), oo)
        cu = cu_seqlens_tensor(seqlens, DEV)
        sp = splits or qfa.fp8_varlen_attn_auto_splits(B, T, H)
        assert sp > 1
        want = qfa.fp8_varlen_attn_split(q8, k8, v8, qfa.descale(st), cu, H, num_splits=sp)
        got = torch.full_like(want, float("nan"))
        assert _call_noalloc(q8, k8, v8, qfa.descale(st), cu, B, T, H, splits, got) == 0, qfa.raw_library().qfa_last_error()
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), (seqlens, H, splits)
        ref, mag = oracle.attention(*o8[:3], o8[3], np.concatenate([[0], np.cumsum(seqlens)]), magnitude=True)
        assert_fp8_attn_close(bf16_to_f32(got), ref, f"no-alloc seqlens {seqlens}", mag=mag)


def test_noalloc_refuses_a_request_beyond_its_workspace():
    e = torch.zeros((1, 1, 128), dtype=torch.uint8, device=DEV)
    o = torch.zeros((1, 1, 128), dtype=torch.bfloat16, device=DEV)
    sc = torch.ones(3, dtype=torch.float32, device=DEV)
    cu = torch.tensor([0, 1], dtype=torch.int32, device=DEV)
    lib = qfa.raw_library()
    # sizes only: the refusal comes before anything is enqueued, so the small tensors are never read
    status = lib.qfa_fp8_varlen_attn_split_noalloc(e.data_ptr(), e.data_ptr(), e.data_ptr(), sc.data_ptr(),
                                                   cu.data_ptr(), 1, 99504, 16, 128, 16, o.data_ptr(), None)
    assert status == 11
