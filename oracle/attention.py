"""Softmax attention over packed variable-length sequences -- test infrastructure only.

"FP8 vision encoder attention" (Requirements) runs FP8 varlen attention with
per-tensor scales over packed variable-length image batches; "FP8 ViT
Encoder Attention" (intro, note) applies it to ViT encoder attention of
single- and multi-image requests.  Readings taken where the pages are silent:
non-causal attention, softmax scale ``1/sqrt(head_dim)``,
attention only within each sequence ``[cu_seqlens[b], cu_seqlens[b+1])``,
tensors laid out ``[tokens, heads, head_dim]``.

The oracle dequantizes the same E4M3 codes the GPU consumes
(``decode(code) * scale`` in float64) and evaluates the plain definition in
float64: ``S = Q K^T / sqrt(D)``, a row softmax with its maximum subtracted,
``O = P V``.

``attention_float`` / ``attention_float_rows`` evaluate the same definition
on real-valued inputs (the bf16 Q, K, V of the BF16 baseline that "FP8 ViT
Encoder Attention", Performance, and "FP8 vision encoder attention",
Expected performance, compare FP8 against).
"""

import math

import numpy as np

from .e4m3 import decode


def _check_cu(cu_seqlens, total_tokens):
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 2 or cu[0] != 0 or cu[-1] != total_tokens or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0, end at the token count and not decrease")
    return cu


def _dequant(codes, scale):
    return decode(codes) * float(scale)


def _softmax_rows(s):
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    return p / p.sum(axis=-1, keepdims=True)


def _attend(qf, kf, vf, magnitude):
    """One sequence and head, float64: (P V, P |V| or None)."""
    p = _softmax_rows(qf @ kf.T * (1.0 / math.sqrt(qf.shape[-1])))
    return p @ vf, (p @ np.abs(vf) if magnitude else None)


def attention_float(q, k, v, cu_seqlens, magnitude=False):
    """Full output, float64 ``[T, H, D]``, from real-valued ``[T, H, D]`` inputs (e.g. bf16 values)."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    T, H, D = q.shape
    cu = _check_cu(cu_seqlens, T)
    out = np.zeros((T, H, D), dtype=np.float64)
    mag = np.zeros((T, H, D), dtype=np.float64) if magnitude else None
    for b in range(cu.size - 1):
        lo, hi = int(cu[b]), int(cu[b + 1])
        for h in range(H):
            if hi == lo:
                continue
            o, m = _attend(q[lo:hi, h], k[lo:hi, h], v[lo:hi, h], magnitude)
            out[lo:hi, h] = o
            if magnitude:
                mag[lo:hi, h] = m
    return (out, mag) if magnitude else out


def attention_float_rows(q, k, v, cu_seqlens, rows, magnitude=False):
    """Output rows ``rows`` (global token indices) of ``attention_float`` only."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    T, H, D = q.shape
    cu = _check_cu(cu_seqlens, T)
    rows = np.asarray(rows, dtype=np.int64)
    seq_of = np.searchsorted(cu, rows, side="right") - 1
    out = np.zeros((rows.size, H, D), dtype=np.float64)
    mag = np.zeros((rows.size, H, D), dtype=np.float64) if magnitude else None
    for b in np.unique(seq_of):
        lo, hi = int(cu[b]), int(cu[b + 1])
        sel = np.nonzero(seq_of == b)[0]
        for h in range(H):
            o, m = _attend(q[rows[sel], h], k[lo:hi, h], v[lo:hi, h], magnitude)
            out[sel, h] = o
            if magnitude:
                mag[sel, h] = m
    return (out, mag) if magnitude else out


def attention(q8, k8, v8, descale, cu_seqlens, magnitude=False):
    """Full output, float64 ``[T, H, D]``, from uint8 codes ``[T, H, D]``.

    With ``magnitude=True`` also returns ``M = P |V|`` (same shape): for each
    output element, the probability-weighted mean magnitude of the values it
    averages.  The tests use it as the element's scale when comparing.
    """
    T, H, D = q8.shape
    cu = _check_cu(cu_seqlens, T)
    out = np.zeros((T, H, D), dtype=np.float64)
    mag = np.zeros((T, H, D), dtype=np.float64) if magnitude else None
    inv_sqrt_d = 1.0 / math.sqrt(D)
    for b in range(cu.size - 1):
        lo, hi = int(cu[b]), int(cu[b + 1])
        if hi == lo:
            continue
        for h in range(H):
            qf = _dequant(q8[lo:hi, h], descale[0])
            kf = _dequant(k8[lo:hi, h], descale[1])
            vf = _dequant(v8[lo:hi, h], descale[2])
            p = _softmax_rows(qf @ kf.T * inv_sqrt_d)
            out[lo:hi, h] = p @ vf
            if magnitude:
                mag[lo:hi, h] = p @ np.abs(vf)
    return (out, mag) if magnitude else out


def attention_rows(q8, k8, v8, descale, cu_seqlens, rows, magnitude=False) -> np.ndarray:
    """Output rows ``rows`` (global token indices) only: float64 ``[len(rows), H, D]``.

    Each query row attends to every key of its own sequence, as in
    ``attention``; this evaluates the same definition for a subset of rows.
    ``magnitude`` as in ``attention``.
    """
    T, H, D = q8.shape
    cu = _check_cu(cu_seqlens, T)
    rows = np.asarray(rows, dtype=np.int64)
    seq_of = np.searchsorted(cu, rows, side="right") - 1
    out = np.zeros((rows.size, H, D), dtype=np.float64)
    mag = np.zeros((rows.size, H, D), dtype=np.float64) if magnitude else None
    inv_sqrt_d = 1.0 / math.sqrt(D)
    for b in np.unique(seq_of):
        lo, hi = int(cu[b]), int(cu[b + 1])
        sel = np.nonzero(seq_of == b)[0]
        for h in range(H):
            qf = _dequant(q8[rows[sel], h], descale[0])
            kf = _dequant(k8[lo:hi, h], descale[1])
            vf = _dequant(v8[lo:hi, h], descale[2])
            p = _softmax_rows(qf @ kf.T * inv_sqrt_d)
            out[sel, h] = p @ vf
            if magnitude:
                mag[sel, h] = p @ np.abs(vf)
    return (out, mag) if magnitude else out
