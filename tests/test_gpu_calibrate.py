"""GPU: calibrate once with dynamic scaling, save the scale file, reload as static scales.

Pages: "FP8 ViT Encoder Attention", Calibrate-Once, Reuse Workflow and Scale
File Format; "FP8 vision encoder attention", Create static scales.  The
library's exported values, the written file and the codes of a static forward
after reloading are compared bit-exactly with the oracle, which sees only the
same bf16 inputs copied to the host.
"""

import numpy as np
import pytest
import torch

import oracle
import quantized_flash_attn_amd as qfa
from helpers import bf16_to_f32, codes, log
from quantized_flash_attn_amd import scale_file as sf
from workloads import WORKLOADS, make_qkv

pytestmark = pytest.mark.gpu

DEV = "cuda"

# Two layers with different statistics: the kernel-benchmark recipe cut to
# 1024 tokens (x20 outliers, per-head sigma) and the tiny 256-token recipe.
LAYERS = {
    "visual.blocks.0.attn.attn": (WORKLOADS[3], 1024, 20),   # 20 forwards: the ring wraps
    "visual.blocks.1.attn.attn": (WORKLOADS[1], None, 16),
}


def test_calibrate_save_load_static(tmp_path):
    states, ostates = {}, {}
    for layer, (w, T, n_fwd) in LAYERS.items():
        log(f"calibrating {layer}: {w.name}, tokens {T or w.total_tokens}, {n_fwd} forwards")
        st = qfa.init_scale_state(DEV)
        ost = oracle.ScaleState()
        for f in range(n_fwd):
            q, k, v = make_qkv(w, f, device=DEV, num_tokens=T)
            qfa.quantize_qkv(st, "dynamic", q, k, v)
            ost.forward_dynamic([oracle.amax(bf16_to_f32(x)) for x in (q, k, v)])
        states[layer], ostates[layer] = st, ost

    # too few forwards are refused before anything is written
    with pytest.raises(ValueError):
        sf.calibrated_scales(states, 1.5, min_forwards=17)

    path = str(tmp_path / "scales.json")
    written = sf.calibrate_to_file(path, states, margin=1.5)
    loaded = sf.load_scale_file(path)
    for layer in LAYERS:
        want = ostates[layer].export_static_amax(1.5)
        assert np.array_equal(np.array(written[layer], np.float32), want), layer
        assert np.array_equal(np.array(loaded[layer], np.float32), want), layer
        log(f"  {layer}: saved amax {want.tolist()}")

    # reload as static scales and run a fresh forward
    for layer, (w, T, n_fwd) in LAYERS.items():
        st = sf.init_scale_state_from_file(path, layer, device=DEV)
        q, k, v = make_qkv(w, n_fwd + 3, device=DEV, num_tokens=T)
        q8, k8, v8 = qfa.quantize_qkv(st, "static", q, k, v)
        snap = qfa.read_scale_state(st)
        ost = oracle.ScaleState(static_amax=ostates[layer].export_static_amax(1.5), margin=1.0)
        descale, inv = ost.forward_static()
        # same scales as loading the raw ring maximum with the margin applied at load
        d2, _ = oracle.ScaleState(static_amax=ostates[layer].ring.max(axis=1), margin=1.5).forward_static()
        assert np.array_equal(descale, d2)
        assert np.array_equal(np.array(snap["descale"], np.float32), descale), layer
        assert snap["cursor"] == 0
        for t, (x, c) in enumerate(zip((q, k, v), (q8, k8, v8))):
            want = oracle.quantize(bf16_to_f32(x), inv[t])
            assert np.array_equal(codes(c), want), (layer, "qkv"[t])


def test_export_refuses_fresh_state():
    st = qfa.init_scale_state(DEV)
    with pytest.raises(qfa.QfaError) as ei:
        qfa.export_static_amax(st, 1.5)
    assert ei.value.status == 8
