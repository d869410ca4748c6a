"""Test-side helpers: host copies of device tensors, the attention tolerance,
and a threaded driver for the oracle's attention on large row sets.

Tolerance (floating point, attention output).  With ``r`` the oracle's
float64 output and ``g`` the kernel's bf16 output, the contract's measure is

    e = |g - r| / max(u, |r|),    pass iff max(e) <= 3e-2 and mean(e) <= 3e-3,

where ``u`` is the output scale: 1 for unit-scale outputs (every workload and
every test whose V is drawn at unit scale), so ``e`` is the absolute error
where |r| <= 1 and the relative error above it (outputs reach ~100 where V
has x20-x30 outliers, where bf16 rounding alone exceeds 3e-2 in absolute
terms).  A test that scales V by a factor passes that factor as ``u``: the
check is then the unit-scale check of the outputs divided by it.

Besides the contract's bound, each kernel has a tighter bound derived from
its own arithmetic, stated on ``e_M = |g - r| / max(u, M)`` with
``M = P|V|`` (the probability-weighted magnitude of the values an output
averages): any finite-precision evaluation of sum_j p_j v_j errs in
proportion to sum_j p_j |v_j|, not to |sum_j p_j v_j|.
"""

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle

TOL_MAX = 3e-2
TOL_MEAN = 3e-3

# E4M3 kernel (fp16 operands, fp32 accumulation, bf16 output).  Q K^T sums
# products of two E4M3 values (at most 8 significant bits each) in fp32, so
# the logits carry only fp32 rounding (relative ~2^-22 on p).  p is rounded
# to fp16 (11 significant bits): p_j(1 + d_j), |d_j| <= 2^-11, and l is the
# sum of the same rounded p, so O / l is an exact convex combination of V
# rows whose weights moved by sum_j (p_j / l) d_j (v_j - O): at most
# 2^-11 (M + |O|) <= 2^-10 M.  The bf16 output adds at most 2^-8 |O| <= 2^-8 M.
# So e_M <= 2^-10 + 2^-8 ~= 4.9e-3, plus fp32 accumulation terms near 2^-16.
# Mean: rounding to bf16 errs by half a spacing at most and a quarter on
# average, a spacing being 2^-7..2^-8 of |O|, so the output term averages at
# most 2^-9 M; the weight term averages well below its 2^-11 scale.  Mean
# e_M <= 2^-9 + 2^-11 ~= 2.4e-3.
TOL_MAX_FP8_M = 6e-3
TOL_MEAN_FP8_M = 2.5e-3

# BF16 baseline attention (bf16 inputs, fp32 products and sums, P rounded to
# bf16, bf16 output).  Rounding P to bf16 (8 significant bits) moves the
# numerator by at most 2^-8 M / l relative to the fp32 denominator, and the
# bf16 output adds at most 2^-8 |r| <= 2^-8 M; the fp32 products, sums and
# exp2 add terms near 2^-20.  So e_M <= 2^-7 ~= 7.8e-3.  Mean: at most
# 2^-9 M from the output rounding (as above) and 2^-9 M from the weights.
TOL_MAX_BF16 = 1e-2
TOL_MEAN_BF16 = 4e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_to_f32(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> float32 numpy array with the same values."""
    return t.detach().to("cpu").float().numpy()


def codes(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").numpy()


def attn_errors(g, r, scale=None, unit=1.0):
    """(max e, mean e) with e = |g - r| / max(unit, scale); scale defaults to |r|."""
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    s = np.abs(r) if scale is None else np.asarray(scale, dtype=np.float64)
    e = np.abs(g - r) / np.maximum(float(unit), s)
    return float(e.max()), float(e.mean())


def one_token_row(v_codes, s_v) -> torch.Tensor:
    """The bf16 output of a one-token sequence, from its V codes (any shape) and s_v: fp32(v * s_v) rounded to
    bf16, with a zero as +0.  The output is a sum of p * v terms that starts from +0 (in the kernels and in the
    oracle alike), so a code of -0 comes out as +0."""
    v = oracle.decode(np.asarray(v_codes)).astype(np.float32) * np.float32(s_v)
    return torch.from_numpy(v + np.float32(0.0)).to(torch.bfloat16)


def check_rows(w):
    """Query rows checked against the oracle at full size: every row, or the
    workload's stated row ranges in full."""
    if not w.oracle_rows:
        return np.arange(w.total_tokens)
    return np.unique(np.concatenate([np.arange(lo, hi) for lo, hi in w.oracle_rows]))


def host_workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_attention_rows(q8, k8, v8, descale, cu, rows, block=1024, workers=None, codes=True):
    """oracle.attention_rows(..., magnitude=True) over many rows (with codes=False:
    oracle.attention_float_rows on real-valued q, k, v, descale unused), run as
    independent (sequence, head, block of rows) pieces on a thread pool.

    Each piece is one call of the oracle on the head's slice; the pieces do not
    interact (softmax rows are independent), so the result equals one call over
    all rows and heads.  Returns (out, mag), float64 [len(rows), H, D].
    """
    cu = np.asarray(cu, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    H, D = q8.shape[1], q8.shape[2]
    out = np.zeros((rows.size, H, D), dtype=np.float64)
    mag = np.zeros_like(out)
    seq_of = np.searchsorted(cu, rows, side="right") - 1
    jobs = []
    for b in np.unique(seq_of):
        sel = np.nonzero(seq_of == b)[0]
        for h in range(H):
            for i in range(0, sel.size, block):
                jobs.append((h, sel[i:i + block]))

    def run(job):
        h, sel = job
        qs, ks, vs = q8[:, h:h + 1], k8[:, h:h + 1], v8[:, h:h + 1]
        if codes:
            o, m = oracle.attention_rows(qs, ks, vs, descale, cu, rows[sel], magnitude=True)
        else:
            o, m = oracle.attention_float_rows(qs, ks, vs, cu, rows[sel], magnitude=True)
        out[sel, h] = o[:, 0]
        mag[sel, h] = m[:, 0]

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:   # pragma: no cover
        threadpool_limits = None
    n = workers or host_workers()
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            with ThreadPoolExecutor(max_workers=n) as ex:
                list(ex.map(run, jobs))
    else:
        with ThreadPoolExecutor(max_workers=n) as ex:
            list(ex.map(run, jobs))
    return out, mag


def assert_attn_close(g, r, what="", mag=None, unit=1.0, tol_max=TOL_MAX, tol_mean=TOL_MEAN, derived=None):
    """Check the kernel's output g against the oracle's r (see the module docstring).

    Asserts the contract's bound on e = |g - r| / max(unit, |r|).  ``mag`` is
    the oracle's M = P|V| for the same elements; with it, e_M is logged and,
    if ``derived`` = (max, mean) is given, asserted too.
    """
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    mx, mean = attn_errors(g, r, unit=unit)
    msg = f"  {what}: e/max({unit:g},|r|) max {mx:.3e} mean {mean:.3e}"
    mx_m = mean_m = None
    if mag is not None:
        mx_m, mean_m = attn_errors(g, r, mag, unit=unit)
        msg += f" | e/max({unit:g},P|V|) max {mx_m:.3e} mean {mean_m:.3e}"
    log(msg)
    assert mx <= tol_max and mean <= tol_mean, f"{what}: contract e max {mx:.3e}, mean {mean:.3e}"
    if derived is not None and mag is not None:
        assert mx_m <= derived[0] and mean_m <= derived[1], \
            f"{what}: e_M max {mx_m:.3e}, mean {mean_m:.3e} above the kernel's derived bound {derived}"


def assert_fp8_attn_close(g, r, what="", mag=None, unit=1.0):
    """The contract's bound plus the E4M3 kernel's derived bound."""
    assert_attn_close(g, r, what, mag=mag, unit=unit, derived=(TOL_MAX_FP8_M, TOL_MEAN_FP8_M))
