"""Quantization of Q, K and V to E4M3 codes -- test infrastructure only.

"FP8 ViT Encoder Attention" (intro) quantizes Q/K/V on the fly to FP8 before
the attention call; its Usage and Calibrate-Once sections say where the scales
come from (see ``oracle.scales``).  Each element becomes
``encode(fp32(fp32(x) * inv[t]))``: one float32 multiply, rounded to nearest
even, then the saturating E4M3 encoding of ``oracle.e4m3``.

``quantize_qkv_packed`` takes the fused QKV projection output ``[T, 3, H, D]``
("FP8 ViT Encoder Attention", Performance, counts the split into three
quantization launches and the head-dim un-padding among the overheads) and
returns codes padded with zeros to 128 dims; the amax covers the D real dims.
"""

import numpy as np

from .e4m3 import encode
from .scales import amax


def quantize(x, inv) -> np.ndarray:
    """float32 array (bf16 values) and one float32 factor -> uint8 codes, same shape."""
    y = (np.asarray(x, dtype=np.float32) * np.float32(inv)).astype(np.float32)
    return encode(y)


def quantize_qkv(state, mode: str, q, k, v) -> tuple:
    """One forward of the quantizer on float32 arrays holding bf16 values.

    ``mode`` is "dynamic" (observe amax, update the ring, then quantize) or
    "static" (loaded scales times margin).  Returns ``(q8, k8, v8, descale,
    observed)`` where ``observed`` is the per-tensor amax this forward saw
    (recorded only in dynamic mode).
    """
    observed = np.array([amax(q), amax(k), amax(v)], dtype=np.float32)
    if mode == "dynamic":
        descale, inv = state.forward_dynamic(observed)
    elif mode == "static":
        descale, inv = state.forward_static()
    else:
        raise ValueError("mode must be 'dynamic' or 'static'")
    return quantize(q, inv[0]), quantize(k, inv[1]), quantize(v, inv[2]), descale, observed


PADDED_DIM = 128


def quantize_qkv_packed(state, mode: str, qkv) -> tuple:
    """One forward on a float32 array ``[T, 3, H, D]`` of bf16 values (D <= 128).

    Q, K, V are ``qkv[:, 0]``, ``qkv[:, 1]``, ``qkv[:, 2]``.  Returns ``(q8, k8,
    v8, descale, observed)`` with codes ``[T, H, 128]`` whose dims past D are 0.
    """
    qkv = np.asarray(qkv, dtype=np.float32)
    T, three, H, D = qkv.shape
    if three != 3 or D > PADDED_DIM:
        raise ValueError("qkv must be [T, 3, H, D] with D <= 128")
    q8, k8, v8, descale, observed = quantize_qkv(state, mode, qkv[:, 0], qkv[:, 1], qkv[:, 2])
    padded = []
    for c in (q8, k8, v8):
        p = np.zeros((T, H, PADDED_DIM), dtype=np.uint8)
        p[:, :, :D] = c
        padded.append(p)
    return padded[0], padded[1], padded[2], descale, observed
