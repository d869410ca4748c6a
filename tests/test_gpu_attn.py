"""GPU parity of the varlen FP8 attention against the oracle.

The GPU runs the whole path through the C ABI (quantize, then attention on
its own codes and scales); the oracle runs its own path (quantize, then
float64 attention) on host copies of the same bf16 inputs.  Codes must agree
bit-exactly; outputs within the contract's tolerance and the kernel's own
derived bound, both stated in tests/helpers.py.
"""

import time

import numpy as np
import pytest
import torch

import oracle
import quantized_flash_attn_amd as qfa
from helpers import (assert_fp8_attn_close, bf16_to_f32, check_rows, codes, log, one_token_row,
                     oracle_attention_rows)
from workloads import WORKLOADS, cu_seqlens_tensor, make_qkv, ramp_qkv, random_qkv

pytestmark = pytest.mark.gpu

DEV = "cuda"


def gpu_path(q, k, v, seqlens, state=None, mode="dynamic"):
    st = state if state is not None else qfa.init_scale_state(DEV)
    q8, k8, v8 = qfa.quantize_qkv(st, mode, q, k, v)
    cu = cu_seqlens_tensor(seqlens, DEV)
    qfa.check_cu_seqlens(cu, q.shape[0])
    out = qfa.fp8_varlen_attn(q8, k8, v8, qfa.descale(st), cu, q.shape[1])
    return (q8, k8, v8), out, st


def oracle_path(q, k, v, seqlens, ost=None, mode="dynamic"):
    ost = ost if ost is not None else oracle.ScaleState()
    qh, kh, vh = (bf16_to_f32(t) for t in (q, k, v))
    q8, k8, v8, descale, _ = oracle.quantize_qkv(ost, mode, qh, kh, vh)
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    return (q8, k8, v8), oracle.attention(q8, k8, v8, descale, cu, magnitude=True), descale


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
    log(f"seqlens={seqlens} H={H} sigma={sigma}")
    q, k, v = random_qkv(seqlens, H, seed=sum(seqlens) * 7 + H, device=DEV, sigma=sigma, outlier_p=outliers,
                         outlier_scale=20.0)
    gcodes, out, _ = gpu_path(q, k, v, seqlens)
    ocodes, (ref, mag), _ = oracle_path(q, k, v, seqlens)
    for g, o in zip(gcodes, ocodes):
        assert np.array_equal(codes(g), o)
    assert_fp8_attn_close(bf16_to_f32(out), ref, f"seqlens {seqlens}", mag=mag)


@pytest.mark.parametrize("order,gain", [("increasing", 4.0), ("decreasing", 4.0), ("increasing", 1.6),
                                        ("increasing", 1.8), ("increasing", 2.0)])
def test_running_max_moves(order, gain):
    """Logits rising along the keys move the running row max, and rescale O
    and l, at every key tile, the ragged last tile included; falling logits
    never move it after the first tile.  Gains 1.6 to 2.0 make the max grow
    by about 7 to 9 log2 units per tile, around the point where p against
    the old max would leave fp16's range."""
    seqlens = [1000, 333, 129]
    log(f"{order} logits, gain {gain}, seqlens={seqlens}")
    q, k, v = ramp_qkv(seqlens, 2, seed=29, device=DEV, order=order, gain=gain)
    gcodes, out, _ = gpu_path(q, k, v, seqlens)
    ocodes, (ref, mag), _ = oracle_path(q, k, v, seqlens)
    for g, o in zip(gcodes, ocodes):
        assert np.array_equal(codes(g), o)
    assert_fp8_attn_close(bf16_to_f32(out), ref, f"{order} logits", mag=mag)


def test_many_short_sequences():
    """About 1500 sequences of 0..40 tokens with a few longer ones: many
    sequences per query tile range, empty sequences, and one spare virtual
    tile per sequence in the tile -> sequence search."""
    g = np.random.default_rng(37)
    seqlens = [int(n) for n in g.integers(0, 41, size=1500)]
    for pos, n in ((100, 257), (700, 513), (1400, 300)):
        seqlens[pos] = n
    log(f"{len(seqlens)} sequences, {sum(seqlens)} tokens")
    q, k, v = random_qkv(seqlens, 2, seed=41, device=DEV, sigma=1.5, outlier_p=0.001, outlier_scale=20.0)
    gcodes, out, _ = gpu_path(q, k, v, seqlens)
    ocodes, (ref, mag), _ = oracle_path(q, k, v, seqlens)
    for gc, oc in zip(gcodes, ocodes):
        assert np.array_equal(codes(gc), oc)
    assert_fp8_attn_close(bf16_to_f32(out), ref, "many short sequences", mag=mag)


def test_max_heads():
    """The largest head count the ABI accepts (65536: a 128-row tile of one
    head then spans just under 2^31 bytes in the buffer descriptors), with
    sequences of 2 and 1 tokens.  The oracle derives the scales from the full
    tensors; codes and outputs are compared on a sample of heads (the first
    and last 256 and 512 drawn at random)."""
    seqlens, H = [2, 1], 65536
    log(f"seqlens={seqlens} H={H}")
    q, k, v = random_qkv(seqlens, H, seed=43, device=DEV, sigma=1.5)
    gcodes, out, st = gpu_path(q, k, v, seqlens)
    qh, kh, vh = (bf16_to_f32(t) for t in (q, k, v))
    ost = oracle.ScaleState()
    descale, inv = ost.forward_dynamic(np.array([oracle.amax(x) for x in (qh, kh, vh)], dtype=np.float32))
    assert np.array_equal(np.array(qfa.read_scale_state(st)["descale"], dtype=np.float32), descale)
    heads = np.unique(np.concatenate([np.arange(256), np.arange(H - 256, H),
                                      np.random.default_rng(43).integers(0, H, size=512)]))
    ocodes = [oracle.quantize(x[:, heads], inv[t]) for t, x in enumerate((qh, kh, vh))]
    for g, o in zip(gcodes, ocodes):
        assert np.array_equal(codes(g)[:, heads], o)
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    ref, mag = oracle.attention(*ocodes, descale, cu, magnitude=True)
    assert_fp8_attn_close(bf16_to_f32(out)[:, heads], ref, f"{H} heads", mag=mag)


def test_distinct_tensor_scales():
    """Very different Q, K, V ranges: the three scales must each go to the right place.

    V is drawn at 100 times unit scale, so the outputs are too: the check is
    the unit-scale check of the outputs divided by 100 (unit=100)."""
    seqlens = [200, 77]
    q, k, v = random_qkv(seqlens, 2, seed=5, device=DEV)
    q, k, v = q * 0.01, k * 30.0, v * 100.0
    _, out, _ = gpu_path(q, k, v, seqlens)
    _, (ref, mag), _ = oracle_path(q, k, v, seqlens)
    assert_fp8_attn_close(bf16_to_f32(out), ref, "distinct scales", mag=mag, unit=100.0)


def test_static_scales_attention():
    seqlens = [300, 129]
    q, k, v = random_qkv(seqlens, 2, seed=9, device=DEV, sigma=2.0)
    sa = [5.0, 7.0, 3.0]
    st = qfa.init_scale_state(DEV, static_amax=sa, margin=1.5)
    _, out, _ = gpu_path(q, k, v, seqlens, state=st, mode="static")
    _, (ref, mag), _ = oracle_path(q, k, v, seqlens, ost=oracle.ScaleState(static_amax=sa, margin=1.5), mode="static")
    assert_fp8_attn_close(bf16_to_f32(out), ref, "static", mag=mag)


def test_one_token_sequence_returns_v_row():
    """A one-key softmax weight is exactly 1: p = 2^8 and l = 2^8 exactly, so the
    output row is bf16(fp32(v8 * s_v)) bit for bit."""
    seqlens = [5, 1, 9, 1]
    q, k, v = random_qkv(seqlens, 2, seed=13, device=DEV, sigma=2.0)
    (q8, k8, v8), out, st = gpu_path(q, k, v, seqlens)
    s_v = np.float32(qfa.read_scale_state(st)["descale"][2])
    for row in (5, 15):
        want_bf16 = one_token_row(codes(v8)[row], s_v)
        got = out[row].cpu()
        log(f"  row {row}: {int((got.view(torch.int16) == want_bf16.view(torch.int16)).sum())} of {got.numel()} "
            "bit-equal")
        assert torch.equal(got.view(torch.int16), want_bf16.view(torch.int16)), row


def test_one_token_row_with_negative_zero_codes():
    """V codes of -0 (tiny negative inputs) in a one-token sequence: the output is a sum of p * v terms that starts
    from +0, as in the oracle, so those dims come out +0 and the rest bit for bit; both entry points."""
    seqlens = [3, 1]
    q, k, v = random_qkv(seqlens, 2, seed=21, device=DEV, sigma=2.0)
    v[3, :, :8] = -1e-30   # far below the smallest E4M3 step at this scale: code 0x80
    st = qfa.init_scale_state(DEV)
    q8, k8, v8 = qfa.quantize_qkv(st, "dynamic", q, k, v)
    assert (codes(v8)[3, :, :8] == 0x80).all()
    s_v = qfa.read_scale_state(st)["descale"][2]
    want = one_token_row(codes(v8)[3], s_v)
    assert not torch.signbit(want[:, :8]).any()
    cu = cu_seqlens_tensor(seqlens, DEV)
    ref = oracle.attention(codes(q8), codes(k8), codes(v8), np.array(qfa.read_scale_state(st)["descale"], np.float32),
                           np.concatenate([[0], np.cumsum(seqlens)]))
    assert not np.signbit(ref[3, :, :8]).any()
    for fn in (qfa.fp8_varlen_attn, qfa.fp8_varlen_attn_fp8qk):
        out = fn(q8, k8, v8, qfa.descale(st), cu, 2)
        assert torch.equal(out[3].cpu().view(torch.int16), want.view(torch.int16)), fn.__name__


def test_identical_keys_give_mean_of_v():
    seqlens = [300]
    q, k, v = random_qkv(seqlens, 2, seed=17, device=DEV)
    k = k[:1].expand_as(k).contiguous()
    (_, _, v8), out, st = gpu_path(q, k, v, seqlens)
    s_v = qfa.read_scale_state(st)["descale"][2]
    vf = oracle.decode(codes(v8)) * s_v
    mean_v, mean_abs_v = vf.mean(axis=0), np.abs(vf).mean(axis=0)
    assert_fp8_attn_close(bf16_to_f32(out), np.broadcast_to(mean_v, out.shape), "identical keys",
                          mag=np.broadcast_to(mean_abs_v, out.shape))


def test_no_leakage_and_determinism():
    seqlens = [300, 129, 64, 500]
    q, k, v = random_qkv(seqlens, 2, seed=19, device=DEV)
    st = qfa.init_scale_state(DEV, static_amax=[8.0, 8.0, 8.0], margin=1.0)   # fixed scales for both runs
    (q8, k8, v8), out1, _ = gpu_path(q, k, v, seqlens, state=st, mode="static")
    out2 = qfa.fp8_varlen_attn(q8, k8, v8, qfa.descale(st), cu_seqlens_tensor(seqlens, DEV), 2)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16)), "not deterministic"
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    k2, v2 = k.clone(), v.clone()
    k2[cu[1]:cu[2]] = torch.randn_like(k2[cu[1]:cu[2]].float()).to(torch.bfloat16) * 5
    v2[cu[1]:cu[2]] = torch.randn_like(v2[cu[1]:cu[2]].float()).to(torch.bfloat16) * 5
    _, out3, _ = gpu_path(q, k2, v2, seqlens, state=st, mode="static")
    for b in (0, 2, 3):
        assert torch.equal(out1[cu[b]:cu[b + 1]].view(torch.int16), out3[cu[b]:cu[b + 1]].view(torch.int16)), b
    assert not torch.equal(out1[cu[1]:cu[2]], out3[cu[1]:cu[2]])


def test_static_without_scales_is_refused():
    st = qfa.init_scale_state(DEV)
    x = torch.zeros((4, 1, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(qfa.QfaError) as ei:
        qfa.quantize_qkv(st, "static", x, x, x)
    assert ei.value.status == 6


def _workload_cases():
    return [(i, m) for i, w in sorted(WORKLOADS.items()) for m in w.modes]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("widx,mode", _workload_cases())
def test_workload_attention(widx, mode):
    """Full-size workloads in the benchmark's launch configuration, every scaling
    mode the workload runs: codes of every forward's checked rows bit-exact, and
    the last forward's attention on every stated row (all rows of workloads 1-3;
    the row ranges of 4 and 5 in full) vs the oracle."""
    w = WORKLOADS[widx]
    log(f"workload {widx} ({w.name}), mode {mode}")
    if mode == "static":
        cal = make_qkv(w, 0, device=DEV, calibration=True)
        sa = [oracle.amax(bf16_to_f32(t)) for t in cal]
        del cal
        st = qfa.init_scale_state(DEV, static_amax=sa, margin=1.5)
        ost = oracle.ScaleState(static_amax=sa, margin=1.5)
    else:
        st = qfa.init_scale_state(DEV)
        ost = oracle.ScaleState()
    for fwd in range(w.forwards):
        xs = make_qkv(w, fwd, device=DEV)
        gq8, gk8, gv8 = qfa.quantize_qkv(st, mode, *xs)
        if mode == "dynamic":
            _, inv = ost.forward_dynamic([oracle.amax(bf16_to_f32(x)) for x in xs])
        else:
            _, inv = ost.forward_static()
        assert np.array_equal(np.array(qfa.read_scale_state(st)["descale"], np.float32), ost.descale), fwd
        if fwd < w.forwards - 1:
            del xs, gq8, gk8, gv8
    cu_list = w.cu_seqlens
    out = qfa.fp8_varlen_attn(gq8, gk8, gv8, qfa.descale(st), cu_seqlens_tensor(w.seqlens, DEV), w.num_heads)
    torch.cuda.synchronize()
    rows = check_rows(w)
    cu = np.array(cu_list)
    seqs = np.unique(np.searchsorted(cu, rows, side="right") - 1)
    log(f"  checking {rows.size} rows x {w.num_heads} heads in sequences {seqs.tolist()}")
    # oracle codes for the checked query rows and the keys/values of their sequences
    q, k, v = xs
    rows_t = torch.from_numpy(rows).to(DEV)
    oq8 = np.zeros((w.total_tokens, w.num_heads, 128), np.uint8)
    ok8 = np.zeros_like(oq8)
    ov8 = np.zeros_like(oq8)
    oq8[rows] = oracle.quantize(bf16_to_f32(q[rows_t]), inv[0])
    assert np.array_equal(codes(gq8[rows_t]), oq8[rows])
    for b in seqs:
        lo, hi = cu[b], cu[b + 1]
        ok8[lo:hi] = oracle.quantize(bf16_to_f32(k[lo:hi]), inv[1])
        ov8[lo:hi] = oracle.quantize(bf16_to_f32(v[lo:hi]), inv[2])
        assert np.array_equal(codes(gk8[lo:hi]), ok8[lo:hi])
        assert np.array_equal(codes(gv8[lo:hi]), ov8[lo:hi])
    t0 = time.perf_counter()
    ref, mag = oracle_attention_rows(oq8, ok8, ov8, ost.descale, cu, rows)
    log(f"  oracle attention on {rows.size} rows: {time.perf_counter() - t0:.1f} s")
    got = bf16_to_f32(out[rows_t])
    assert_fp8_attn_close(got, ref, f"workload {widx} {mode}", mag=mag)


@pytest.mark.parametrize("seqlens", [[0], [0, 0, 0]])
def test_empty_batch(seqlens):
    """No tokens at all: both attention entries return an empty output and leave the stream usable."""
    H = 2
    cu = cu_seqlens_tensor(seqlens, DEV)
    st = qfa.init_scale_state(DEV)
    e = torch.zeros((0, H, 128), dtype=torch.bfloat16, device=DEV)
    q8, k8, v8 = qfa.quantize_qkv(st, "dynamic", e, e, e)
    out = qfa.fp8_varlen_attn(q8, k8, v8, qfa.descale(st), cu, H)
    assert tuple(out.shape) == (0, H, 128)
    out_b = qfa.bf16_varlen_attn(e, e, e, cu, H)
    assert tuple(out_b.shape) == (0, H, 128)
    # a non-empty call right after still works
    q, k, v = random_qkv([5], H, seed=3, device=DEV)
    gcodes, got, _ = gpu_path(q, k, v, [5])
    ocodes, (ref, mag), _ = oracle_path(q, k, v, [5])
    assert_fp8_attn_close(bf16_to_f32(got), ref, "after empty", mag=mag)
