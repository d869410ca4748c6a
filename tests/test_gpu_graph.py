"""GPU: the whole path captured in a HIP graph and replayed, against eager runs and the oracle.

The dynamic path keeps its ring cursor on the device, so a captured forward
stays correct when replayed: every replay pushes that forward's amax into the
next slot ("FP8 ViT Encoder Attention", Usage: a 16-entry circular buffer of
observed amax values drives per-forward scale updates).  Launch overhead is
what the pages name as the cost of small images ("FP8 ViT Encoder
Attention", Performance), and graph replay removes it.

Each replay is followed by eager work (an eager forward on a second state
fed the same inputs) and a synchronisation, and every replay is checked
bit-exactly: codes, scale state and attention output against the eager run,
and the ring against the oracle.
"""

import numpy as np
import pytest
import torch

import oracle
import quantized_flash_attn_amd as qfa
from helpers import bf16_to_f32, codes, log
from workloads import WORKLOADS, HEAD_DIM, cu_seqlens_tensor, make_qkv

pytestmark = pytest.mark.gpu

DEV = "cuda"

CASES = [
    # (name, recipe, sequence lengths, heads, mode)
    ("tiny image, dynamic", WORKLOADS[1], (256,), 2, "dynamic"),
    ("ragged packed batch, dynamic", WORKLOADS[3], (300, 17, 700, 1), 4, "dynamic"),
    ("mid-size image, static", WORKLOADS[2], (2304,), 16, "static"),
]


def _forward(st, mode, q, k, v, q8, k8, v8, cu, H, out):
    qfa.quantize_qkv(st, mode, q, k, v, q8, k8, v8)
    qfa.fp8_varlen_attn(q8, k8, v8, qfa.descale(st), cu, H, out=out)


@pytest.mark.parametrize("name,w,seqlens,H,mode", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(name, w, seqlens, H, mode):
    T = sum(seqlens)
    log(f"graph case: {name}, T {T}, H {H}, mode {mode}")
    static = [120.0, 110.0, 9.0] if mode == "static" else None

    def state():
        return qfa.init_scale_state(DEV, static_amax=static, margin=1.5)

    def buffers():
        return (torch.empty((T, H, HEAD_DIM), dtype=torch.uint8, device=DEV) for _ in range(3))

    qs, ks, vs = (torch.zeros((T, H, HEAD_DIM), dtype=torch.bfloat16, device=DEV) for _ in range(3))
    q8, k8, v8 = buffers()
    out = torch.empty((T, H, HEAD_DIM), dtype=torch.bfloat16, device=DEV)
    cu = cu_seqlens_tensor(seqlens, DEV)

    # load every kernel once outside the capture, on a throwaway state
    _forward(state(), mode, qs, ks, vs, q8, k8, v8, cu, H, out)
    torch.cuda.synchronize()

    gst, est = state(), state()
    ost = oracle.ScaleState(static_amax=static, margin=1.5) if static else oracle.ScaleState()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _forward(gst, mode, qs, ks, vs, q8, k8, v8, cu, H, out)
    torch.cuda.synchronize()

    eq8, ek8, ev8 = buffers()
    eout = torch.empty_like(out)
    for r in range(5):
        wq = make_qkv(w, r, device=DEV, num_tokens=T)
        wq = tuple(x[:, :H].contiguous() if x.shape[1] != H else x for x in wq)
        for dst, src in zip((qs, ks, vs), wq):
            dst.copy_(src)
        graph.replay()
        torch.cuda.synchronize()
        _forward(est, mode, *wq, eq8, ek8, ev8, cu, H, eout)          # eager work between replays
        torch.cuda.synchronize()
        for g, e, t in zip((q8, k8, v8), (eq8, ek8, ev8), "qkv"):
            assert torch.equal(g, e), (r, t)
        assert torch.equal(out, eout), r
        gs, es = qfa.read_scale_state(gst), qfa.read_scale_state(est)
        assert gs == es, r
        if mode == "dynamic":
            ost.forward_dynamic([oracle.amax(bf16_to_f32(x)) for x in wq])
            assert gs["cursor"] == r + 1
        else:
            ost.forward_static()
            assert gs["cursor"] == 0
        assert np.array_equal(np.array(gs["descale"], np.float32), ost.descale), r
        if mode == "dynamic":
            for t in range(3):
                assert np.array_equal(np.array(gs["ring"][t], np.float32), ost.ring[t]), (r, t)
        # the replay's codes are the oracle's codes for this forward's inputs
        assert np.array_equal(codes(q8), oracle.quantize(bf16_to_f32(wq[0]), ost.inv[0])), r
    log(f"  5 replays bit-identical to eager; cursor {gs['cursor']}")


def test_graph_split_noalloc_replays_match_eager():
    """Quantize + the no-allocation split-key attention captured in one graph: the capture allocates nothing
    (the split workspace is the library's fixed device array), and every replay equals the eager forward bit for
    bit.  2304 tokens x 8 heads, dynamic: the automatic rule splits the keys into 3 ranges."""
    seqlens, H, mode = (2304,), 8, "dynamic"
    T = sum(seqlens)
    assert qfa.fp8_varlen_attn_auto_splits(1, T, H) == 3
    log(f"graph case: split no-allocation attention, T {T}, H {H}, {mode}")
    w = WORKLOADS[3]
    qs, ks, vs = (torch.zeros((T, H, HEAD_DIM), dtype=torch.bfloat16, device=DEV) for _ in range(3))
    q8, k8, v8 = (torch.empty((T, H, HEAD_DIM), dtype=torch.uint8, device=DEV) for _ in range(3))
    out = torch.empty((T, H, HEAD_DIM), dtype=torch.bfloat16, device=DEV)
    cu = cu_seqlens_tensor(seqlens, DEV)

    def forward(st, q, k, v, c8, o):
        qfa.quantize_qkv(st, mode, q, k, v, *c8)
        qfa.fp8_varlen_attn_split_noalloc(*c8, qfa.descale(st), cu, H, out=o)

    forward(qfa.init_scale_state(DEV), qs, ks, vs, (q8, k8, v8), out)   # kernels loaded, workspace address looked up
    torch.cuda.synchronize()
    gst, est = qfa.init_scale_state(DEV), qfa.init_scale_state(DEV)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        forward(gst, qs, ks, vs, (q8, k8, v8), out)
    torch.cuda.synchronize()
    e8 = tuple(torch.empty_like(q8) for _ in range(3))
    eout = torch.empty_like(out)
    for r in range(5):
        wq = tuple(x[:, :H].contiguous() for x in make_qkv(w, r, device=DEV, num_tokens=T))
        for dst, src in zip((qs, ks, vs), wq):
            dst.copy_(src)
        graph.replay()
        torch.cuda.synchronize()
        forward(est, *wq, e8, eout)                                    # eager work on the same workspace
        torch.cuda.synchronize()
        for g, e in zip((q8, k8, v8), e8):
            assert torch.equal(g, e), r
        assert torch.equal(out.view(torch.int16), eout.view(torch.int16)), r
        # and the split merge equals the unsplit kernel on these codes to the FP8 kernel's rounding
        ref = qfa.fp8_varlen_attn(*e8, qfa.descale(est), cu, H)
        torch.cuda.synchronize()
        assert (out.float() - ref.float()).abs().max().item() <= 2e-2 * max(1.0, ref.float().abs().max().item()), r
    log("  5 replays bit-identical to eager")
