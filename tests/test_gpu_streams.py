"""Distinct scale states are independent: the library keeps no device state
of its own (the amax partials live in each state's buffer), so two states
driven at the same time on two streams give, forward by forward, the same
codes and outputs as the same forwards run one after the other.  The kernels
are deterministic (no atomics), so the comparison is bit-exact."""

import pytest
import torch

import quantized_flash_attn_amd as qfa
from helpers import log
from workloads import cu_seqlens_tensor, random_qkv

pytestmark = pytest.mark.gpu

DEV = "cuda"
H = 4


def _forwards(st, inputs, seqlens):
    outs = []
    cu = cu_seqlens_tensor(seqlens, DEV)
    for q, k, v in inputs:
        q8, k8, v8 = qfa.quantize_qkv(st, "dynamic", q, k, v)
        outs.append((q8, k8, v8, qfa.fp8_varlen_attn(q8, k8, v8, qfa.descale(st), cu, H)))
    return outs


def test_two_states_on_two_streams():
    seqlens_a, seqlens_b = [700, 300], [1024]
    # rising sigma makes the first forwards of state A set new maxima (second quantize pass)
    ins_a = [random_qkv(seqlens_a, H, seed=100 + f, device=DEV, sigma=1.0 + f) for f in range(4)]
    ins_b = [random_qkv(seqlens_b, H, seed=200 + f, device=DEV, sigma=2.0, outlier_p=0.001, outlier_scale=20.0)
             for f in range(4)]
    ref_a = _forwards(qfa.init_scale_state(DEV), ins_a, seqlens_a)
    ref_b = _forwards(qfa.init_scale_state(DEV), ins_b, seqlens_b)
    torch.cuda.synchronize()

    main = torch.cuda.current_stream()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    sa.wait_stream(main)
    sb.wait_stream(main)
    with torch.cuda.stream(sa):
        st_a = qfa.init_scale_state(DEV)
        got_a = _forwards(st_a, ins_a, seqlens_a)
    with torch.cuda.stream(sb):
        st_b = qfa.init_scale_state(DEV)
        got_b = _forwards(st_b, ins_b, seqlens_b)
    torch.cuda.synchronize()

    for name, ref, got in (("A", ref_a, got_a), ("B", ref_b, got_b)):
        for f, (r, g) in enumerate(zip(ref, got)):
            for what, x, y in zip(("q8", "k8", "v8", "out"), r, g):
                assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), f"state {name} forward {f} {what}"
    snap_a, snap_b = qfa.read_scale_state(st_a), qfa.read_scale_state(st_b)
    log(f"state A cursor {snap_a['cursor']}, state B cursor {snap_b['cursor']}")
    assert snap_a["cursor"] == 4 and snap_b["cursor"] == 4
