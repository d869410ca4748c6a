"""GPU parity of amax, ring, scales and E4M3 codes against the oracle (bit-exact).

All calls go through the C ABI (binding in quantized_flash_attn_amd).  The
oracle computes its expected values from the same bf16 inputs, copied to the
host; nothing it uses comes from the HIP path.
"""

import numpy as np
import pytest
import torch

import oracle
import quantized_flash_attn_amd as qfa
from helpers import bf16_to_f32, codes, log
from workloads import WORKLOADS, make_qkv

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _all_bf16_tensor():
    """Every bf16 bit pattern except NaN (NaNs replaced by 0), shape [512, 1, 128]."""
    bits = np.arange(65536, dtype=np.uint32)
    exp = (bits >> 7) & 0xFF
    man = bits & 0x7F
    bits[(exp == 0xFF) & (man != 0)] = 0
    t = torch.from_numpy(bits.astype(np.uint16).view(np.int16).copy()).view(torch.bfloat16).reshape(512, 1, 128)
    return t


def _state_equal(snap, ost, dynamic=True):
    hist = ost.history_len
    for t in range(3):
        want_d, want_i = oracle.scales_from_amax(ost.amax_eff)
        assert np.float32(snap["amax_eff"][t]) == ost.amax_eff[t], ("amax_eff", t)
        assert np.float32(snap["descale"][t]) == want_d[t], ("descale", t)
        assert np.float32(snap["inv"][t]) == want_i[t], ("inv", t)
        if dynamic:
            assert np.array_equal(np.array(snap["ring"][t], np.float32), ost.ring[t][:hist]), ("ring", t)
    if dynamic:
        assert snap["cursor"] == ost.cursor


@pytest.mark.parametrize("static_amax,margin", [
    (448.0, 1.0), (7.0, 1.0), (3.0, 1.0), (1.0, 1.5), (0.1, 1.5), (1e-3, 1.0), (2.0 ** -100, 1.0),
    (1e-35, 1.0), (65504.0, 1.0), (1e30, 1.5), (300.7, 1.5), (224.0, 1.0), (198.0, 1.0),
])
def test_every_bf16_static(static_amax, margin):
    x = _all_bf16_tensor()
    xd = x.to(DEV)
    st = qfa.init_scale_state(DEV, static_amax=[static_amax] * 3, margin=margin)
    q8, k8, v8 = qfa.quantize_qkv(st, "static", xd, xd, xd)
    snap = qfa.read_scale_state(st)
    ost = oracle.ScaleState(static_amax=[static_amax] * 3, margin=margin)
    descale, inv = ost.forward_static()
    _state_equal(snap, ost, dynamic=False)
    assert snap["cursor"] == 0 and all(v == 0.0 for r in snap["ring"] for v in r)
    want = oracle.quantize(bf16_to_f32(x), inv[0])
    for c in (q8, k8, v8):
        got = codes(c)
        bad = np.nonzero(got != want)
        assert bad[0].size == 0, f"{bad[0].size} mismatches, first at {[b[0] for b in bad]}"


def test_dynamic_scales_over_bf16_amax_sweep():
    """Dynamic finalize (history 1) for ~2000 amax values spread over the bf16 range."""
    bits = np.concatenate([np.arange(1, 0x7F80, 16), [1, 2, 0x0D80, 0x0D81, 0x7F7F, 0x3F80, 0x43E0]]).astype(np.uint32)
    vals = (bits << 16).view(np.float32)
    st = qfa.init_scale_state(DEV, history_len=1)
    ost = oracle.ScaleState(history_len=1)
    base = torch.zeros((1, 1, 128), dtype=torch.bfloat16)
    for n, a in enumerate(vals):
        q = base.clone(); q[0, 0, 3] = float(a)
        k = base.clone(); k[0, 0, 100] = -float(a)
        v = base.clone(); v[0, 0, 0] = float(a)
        q8, k8, v8 = qfa.quantize_qkv(st, "dynamic", q.to(DEV), k.to(DEV), v.to(DEV))
        _, inv = ost.forward_dynamic([a, a, a])
        snap = qfa.read_scale_state(st)
        _state_equal(snap, ost)
        assert codes(q8)[0, 0, 3] == oracle.quantize(bf16_to_f32(q), inv[0])[0, 0, 3]
        assert codes(k8)[0, 0, 100] == oracle.quantize(bf16_to_f32(k), inv[1])[0, 0, 100]
    log(f"  {len(vals)} amax values checked")


def test_zero_tiny_and_empty():
    st = qfa.init_scale_state(DEV)
    ost = oracle.ScaleState()
    z = torch.zeros((3, 2, 128), dtype=torch.bfloat16, device=DEV)
    tiny = torch.full((3, 2, 128), 1e-38, dtype=torch.bfloat16, device=DEV)
    q8, k8, v8 = qfa.quantize_qkv(st, "dynamic", z, -z, tiny)
    ost.forward_dynamic([0.0, 0.0, oracle.amax(bf16_to_f32(tiny))])
    _state_equal(qfa.read_scale_state(st), ost)
    assert np.all(codes(q8) == 0) and np.all(codes(k8) == 0x80)
    want_v = oracle.quantize(bf16_to_f32(tiny), ost.inv[2])
    assert np.array_equal(codes(v8), want_v)
    # empty forward: records amax 0
    e = torch.zeros((0, 2, 128), dtype=torch.bfloat16, device=DEV)
    qfa.quantize_qkv(st, "dynamic", e, e, e)
    ost.forward_dynamic([0.0, 0.0, 0.0])
    _state_equal(qfa.read_scale_state(st), ost)


def _check_forward_codes(w, fwd, xs, outs, inv, full):
    """Codes bit-exact: everywhere if ``full``, else on a seeded sample plus both ends."""
    rng = np.random.default_rng(1000 * w.index + fwd)
    for name, x, c, i in zip("qkv", xs, outs, inv):
        xf = x.reshape(-1)
        cg = c.reshape(-1)
        if not full:
            n = xf.numel()
            idx = np.unique(np.concatenate([np.arange(min(n, 65536)), np.arange(max(0, n - 65536), n),
                                            rng.integers(0, n, size=min(n, 1 << 20))]))
            idx = torch.from_numpy(idx).to(xf.device)
            xf, cg = xf[idx], cg[idx]
        got = codes(cg)
        want = oracle.quantize(bf16_to_f32(xf), i)
        bad = np.count_nonzero(got != want)
        assert bad == 0, f"workload {w.index} forward {fwd} tensor {name}: {bad} code mismatches"


@pytest.mark.timeout(600)
@pytest.mark.parametrize("widx", [1, 2, 3, 4, 5])
def test_workload_quantize(widx):
    """Every forward of every workload: amax, ring, scales bit-exact; codes full or sampled."""
    w = WORKLOADS[widx]
    for mode in w.modes:
        log(f"workload {widx} ({w.name}), mode {mode}, {w.forwards} forwards")
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
            outs = qfa.quantize_qkv(st, mode, *xs)
            snap = qfa.read_scale_state(st)
            if mode == "dynamic":
                observed = [oracle.amax(bf16_to_f32(x)) for x in xs]
                _, inv = ost.forward_dynamic(observed)
                assert np.array_equal(np.array(snap["amax_observed"], np.float32), np.array(observed, np.float32))
            else:
                _, inv = ost.forward_static()
            _state_equal(snap, ost, dynamic=(mode == "dynamic"))
            full = w.total_tokens <= 8192 and (fwd in (0, w.forwards - 1) or w.total_tokens <= 2304)
            _check_forward_codes(w, fwd, xs, outs, inv, full)
            del xs, outs
        log(f"  ok: final amax_eff {snap['amax_eff']}")


def _with_amax(shape, amax, seed):
    """bf16 tensor of ``shape`` with values in (-amax/4, amax/4) and one element equal to -amax (so max|x| = amax)."""
    g = torch.Generator().manual_seed(seed)
    x = (torch.rand(shape, generator=g) - 0.5) * (amax / 2)
    x.view(-1)[int(torch.randint(0, x.numel(), (1,), generator=g))] = -amax
    return x.to(torch.bfloat16)


# Per-forward amax of Q, K and V with a ring of 4 slots.  Q walks through: the
# first forward (empty ring), amax below the other slots' maximum, a new
# maximum, that maximum leaving the window (the scale drops with no second
# pass), an amax equal to the other slots' maximum, and a new maximum once more.
_AMAX_SEQ = {
    0: [2.0, 1.0, 1.5, 3.0, 1.0, 2.5, 0.5, 1.0, 2.5, 2.625],
    1: [0.25, 0.5, 1.0, 2.0, 4.0, 8.0, 16.0, 32.0, 64.0, 128.0],
    2: [5.0, 5.0, 5.0, 5.0, 5.0, 5.0, 5.0, 5.0, 5.0, 5.0],
}


def _expected_requant(ost, observed):
    """From the oracle's ring before this forward: a second pass is needed when amax_t exceeds the maximum of the
    slots other than the one this forward replaces (only then does the scale differ from the one known in advance)."""
    keep = np.arange(ost.history_len) != ost.cursor % ost.history_len
    others = ost.ring[:, keep].max(axis=1) if keep.any() else np.zeros(3, np.float32)
    return [int(np.float32(observed[t]) > others[t]) for t in range(3)]


@pytest.mark.parametrize("T,H", [(1, 1), (256, 2), (512, 1), (300, 2), (4096, 16)])
def test_single_pass_and_second_pass(T, H):
    """Codes, ring and scales bit-exact on every forward, whichever pass produced them, and the
    requantized flag as the ring dictates."""
    st = qfa.init_scale_state(DEV, history_len=4)
    ost = oracle.ScaleState(history_len=4)
    seen = set()
    for fwd in range(len(_AMAX_SEQ[0])):
        xs = [_with_amax((T, H, 128), _AMAX_SEQ[t][fwd], seed=31 * fwd + t) for t in range(3)]
        observed = [oracle.amax(bf16_to_f32(x)) for x in xs]
        want_requant = _expected_requant(ost, observed)
        outs = qfa.quantize_qkv(st, "dynamic", *[x.to(DEV) for x in xs])
        _, inv = ost.forward_dynamic(observed)
        snap = qfa.read_scale_state(st)
        _state_equal(snap, ost)
        assert snap["requantized"] == want_requant, (fwd, snap["requantized"], want_requant)
        seen.update(want_requant)
        for t in range(3):
            got = codes(outs[t])
            want = oracle.quantize(bf16_to_f32(xs[t]), inv[t])
            assert np.array_equal(got, want), (fwd, t, int(np.count_nonzero(got != want)))
    assert seen == {0, 1}


@pytest.mark.parametrize("T,H", [(170, 3), (777, 3)])
def test_single_pass_packed(T, H):
    """The same sequence through the fused [T, 3, H, D] entry point (D = 80)."""
    D = 80
    st = qfa.init_scale_state(DEV, history_len=4)
    ost = oracle.ScaleState(history_len=4)
    for fwd in range(len(_AMAX_SEQ[0])):
        xs = [_with_amax((T, H, D), _AMAX_SEQ[t][fwd], seed=77 * fwd + t) for t in range(3)]
        qkv = torch.stack(xs, dim=1).contiguous()
        observed = [oracle.amax(bf16_to_f32(x)) for x in xs]
        want_requant = _expected_requant(ost, observed)
        g = qfa.quantize_qkv_packed(st, "dynamic", qkv.to(DEV))
        o8q, o8k, o8v, descale, _ = oracle.quantize_qkv_packed(ost, "dynamic", bf16_to_f32(qkv))
        snap = qfa.read_scale_state(st)
        assert snap["requantized"] == want_requant, (fwd, snap["requantized"], want_requant)
        assert np.array_equal(np.array(snap["descale"], np.float32), descale)
        for gg, oo in zip(g, (o8q, o8k, o8v)):
            assert np.array_equal(codes(gg), oo), fwd


def test_paths_share_one_state():
    """Forwards of varying size on one state (so a varying number of amax partials per tensor), switching
    between the split and fused entry points: ring, cursor, scales, requantized flags and codes bit-exact
    against the oracle after every forward."""
    st = qfa.init_scale_state(DEV, history_len=4)
    ost = oracle.ScaleState(history_len=4)
    shapes = [(256, 2), (2048, 4), (100, 5), (300, 2), (64, 8), (1000, 1), (512, 1), (4096, 16), (3, 2), (700, 1)]
    for fwd, (T, H) in enumerate(shapes):
        xs = [_with_amax((T, H, 128), _AMAX_SEQ[t][fwd], seed=13 * fwd + t) for t in range(3)]
        observed = [oracle.amax(bf16_to_f32(x)) for x in xs]
        want_requant = _expected_requant(ost, observed)
        if fwd % 3 == 2:
            outs = qfa.quantize_qkv_packed(st, "dynamic", torch.stack(xs, dim=1).contiguous().to(DEV))
        else:
            outs = qfa.quantize_qkv(st, "dynamic", *[x.to(DEV) for x in xs])
        _, inv = ost.forward_dynamic(observed)
        snap = qfa.read_scale_state(st)
        _state_equal(snap, ost)
        assert snap["requantized"] == want_requant, (fwd, T, H, snap["requantized"], want_requant)
        for t in range(3):
            assert np.array_equal(codes(outs[t]), oracle.quantize(bf16_to_f32(xs[t]), inv[t])), (fwd, T, H, t)
