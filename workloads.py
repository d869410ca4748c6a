"""Seeded synthetic ViT-attention workloads (shapes, distributions, seeds).

Shared by the tests, ``bench.py`` and ``__graft_entry__.smoke()``.  It holds
no arithmetic of the method itself (no amax, scales, quantization or
attention): it only draws bf16 Q/K/V tensors and builds ``cu_seqlens``.

The pages measure on real images (HD to 4K, several images per request:
"FP8 ViT Encoder Attention", Performance) and on datasets that are not
available here; these seeded draws stand in for them.  Recipe:

* ``z ~ N(0, 1)`` in float32 from a seeded ``torch.Generator`` on the target
  device, times a per-head sigma broadcast over ``[T, H, D]``;
* outliers: an independent Bernoulli(p) mask per element and tensor scales the
  element by a factor, in float32;
* one cast to bf16 (round to nearest even);
* per-head sigma ~ U(0.5, 3), drawn once per workload from its own seed and
  shared by Q and K (and V where V uses it too);
* seeds: ``1000*workload + 10*forward + {q: 0, k: 1, v: 2}``, calibration draws
  ``+5000``, sigma draws ``+9000``.
"""

from dataclasses import dataclass, field

import torch

HEAD_DIM = 128


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: packed sequence lengths, heads and value recipe."""

    index: int
    name: str
    seqlens: tuple
    num_heads: int
    qk_sigma: str            # "unit" or "per_head"
    v_sigma: str             # "unit" or "per_head"
    outlier_p: float
    outlier_scale: float
    modes: tuple             # scaling modes this workload runs
    forwards: int            # forwards per mode
    oracle_rows: tuple = field(default=())   # (start, stop) row ranges checked in full at full size; () = all rows

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seqlens))

    @property
    def cu_seqlens(self) -> list:
        cu = [0]
        for n in self.seqlens:
            cu.append(cu[-1] + int(n))
        return cu

    @property
    def attn_flop(self) -> int:
        """Algorithmic attention work: two matmuls, 2 flop per multiply-add."""
        return int(sum(4 * n * n * self.num_heads * HEAD_DIM for n in self.seqlens))

    @property
    def exp2_count(self) -> int:
        """Softmax exponentials of the attention: one per (query, key) pair of a sequence, per head."""
        return int(sum(n * n * self.num_heads for n in self.seqlens))


WORKLOADS = {
    1: Workload(1, "tiny single image, 1x256 tokens, 2 heads", (256,), 2, "unit", "unit", 0.005, 30.0,
                ("dynamic",), 3),
    2: Workload(2, "mid-size image, 1x2304 tokens (48x48 patches), 16 heads", (2304,), 16, "per_head", "unit",
                0.0, 1.0, ("static",), 2),
    3: Workload(3, "kernel-benchmark shape, 1x8192 tokens, 16 heads", (8192,), 16, "per_head", "per_head",
                0.001, 20.0, ("dynamic",), 16),
    4: Workload(4, "QHD packed batch, 3x14400 tokens (90x160 patches), 16 heads", (14400, 14400, 14400), 16,
                "per_head", "unit", 0.0, 1.0, ("dynamic", "static"), 3,
                oracle_rows=((0, 14400), (14400 + 12352, 28800), (28800, 28800 + 2048))),
    5: Workload(5, "4K packed ragged batch, 3x32400 + 2304 tokens, 16 heads", (32400, 32400, 32400, 2304), 16,
                "per_head", "per_head", 0.001, 20.0, ("dynamic",), 16,
                oracle_rows=((97200, 99504), (60704, 64800))),
}


def head_sigma(w: Workload) -> torch.Tensor:
    """Per-head sigma ~ U(0.5, 3), float32 [H], from seed 1000*index + 9000."""
    g = torch.Generator(device="cpu")
    g.manual_seed(1000 * w.index + 9000)
    return 0.5 + 2.5 * torch.rand(w.num_heads, generator=g, dtype=torch.float32)


def _draw(shape, sigma_h, outlier_p, outlier_scale, seed, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if sigma_h is not None:
        z.mul_(sigma_h.to(device).view(1, -1, 1))
    if outlier_p > 0.0:
        mask = torch.rand(shape, generator=g, device=device, dtype=torch.float32) < outlier_p
        z = torch.where(mask, z * outlier_scale, z)
    return z.to(torch.bfloat16)


def make_qkv(w: Workload, forward: int, device="cpu", calibration: bool = False, num_tokens=None) -> tuple:
    """bf16 Q, K, V ``[T, H, 128]`` for ``forward`` (0-based) of workload ``w``.

    ``calibration`` selects the separate calibration draw used for static
    scales.  ``num_tokens`` overrides T (small variants for tests).
    """
    T = w.total_tokens if num_tokens is None else int(num_tokens)
    shape = (T, w.num_heads, HEAD_DIM)
    sig = head_sigma(w)
    base = 1000 * w.index + 10 * forward + (5000 if calibration else 0)
    out = []
    for t, which in enumerate(("q", "k", "v")):
        kind = w.v_sigma if which == "v" else w.qk_sigma
        sigma_h = sig if kind == "per_head" else None
        out.append(_draw(shape, sigma_h, w.outlier_p, w.outlier_scale, base + t, device))
    return tuple(out)


def cu_seqlens_tensor(seqlens, device="cpu") -> torch.Tensor:
    cu = [0]
    for n in seqlens:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32, device=device)


def random_qkv(seqlens, num_heads, seed, device="cpu", sigma=1.0, outlier_p=0.0, outlier_scale=1.0) -> tuple:
    """Free-form seeded bf16 Q, K, V for edge-case tests (ragged lengths, few heads)."""
    T = int(sum(seqlens))
    shape = (T, num_heads, HEAD_DIM)
    sig = torch.full((num_heads,), float(sigma), dtype=torch.float32)
    return tuple(_draw(shape, sig, outlier_p, outlier_scale, seed + t, device) for t in range(3))


def ramp_qkv(seqlens, num_heads, seed, device="cpu", order="increasing", gain=4.0) -> tuple:
    """Seeded bf16 Q, K, V whose logits move steadily along each sequence.

    Every query of a head is a small perturbation of one positive direction
    u_h (entries in [1, 2)), and key j of a sequence of n tokens is
    gain * u_h * s_j with s_j rising from 0.05 to 1 over the sequence
    (``order`` "increasing") or falling from 1 to 0.05 ("decreasing").  With
    the default gain of 4 the scaled logits grow by about 18 log2 units per
    128 keys of a 1000-token sequence (faster in shorter ones) for the
    increasing order, more than a running max may lag plus the margin it
    keeps after moving, so the running row max moves at every key tile
    (except a ragged last tile of one key); for the decreasing order it never
    moves after the first tile.  The growth is proportional to the gain:
    gains near 1.8 put it near 8 log2 units per tile.  V is N(0, 1).
    """
    T = int(sum(seqlens))
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    u = 1.0 + torch.rand((num_heads, HEAD_DIM), generator=g)
    q = u.expand(T, num_heads, HEAD_DIM) * (1.0 + 0.05 * torch.randn((T, num_heads, HEAD_DIM), generator=g))
    s = []
    for n in seqlens:
        r = torch.linspace(0.05, 1.0, int(n)) if int(n) > 1 else torch.ones(int(n))
        s.append(r if order == "increasing" else r.flip(0))
    s = torch.cat(s) if s else torch.zeros(0)
    k = gain * u.expand(T, num_heads, HEAD_DIM) * s.view(-1, 1, 1)
    v = torch.randn((T, num_heads, HEAD_DIM), generator=g)
    return tuple(t.to(torch.bfloat16).to(device) for t in (q, k, v))
