"""Per-tensor amax and the per-forward scale state -- test infrastructure only.

Pages (cited by title and section):

* "FP8 ViT Encoder Attention", Usage: with no scale file, dynamic scaling is
  used; a 16-entry circular buffer of observed Q/K/V amax values drives the
  per-forward scale updates.
* "FP8 vision encoder attention", Enable FP8 attention: the observed Q/K/V
  maxima are recorded in a 16-entry circular buffer and the scales are
  updated during each forward pass.
* "FP8 ViT Encoder Attention", Calibrate-Once, Reuse Workflow, and "FP8
  vision encoder attention", Create static scales: saved scales are
  multiplied by a save margin whose default is 1.5; static scales remove the
  dynamic work.

Readings taken where the pages are silent:

* One buffer per tensor (Q, K, V); unfilled slots start at 0, so the maximum
  over all slots is the maximum over the filled ones.
* A forward's own amax counts toward that forward's scale: push, then take
  the maximum, then quantize.
* A stored static scale is an amax (range) value; the effective amax in
  static mode is ``fp32(static_amax) * fp32(margin)`` and the ring is unused.
* The scale learned by calibration ("FP8 ViT Encoder Attention",
  Calibrate-Once, Reuse Workflow; "FP8 vision encoder attention", Create
  static scales) is the ring maximum after the dynamic forwards, and the
  saved value is ``fp32(ring max * margin)``; it is loaded with margin 1.0.
* ``a = max(amax_eff, 2**-100)`` keeps both factors finite for all-zero or
  tiny tensors; ``descale = fp32(a / 448)`` dequantizes and
  ``inv = fp32(448 / a)`` quantizes, each one IEEE float32 division.
"""

from dataclasses import dataclass, field

import numpy as np

HISTORY_LEN = 16
AMAX_FLOOR = np.float32(2.0 ** -100)
_FP8_MAX32 = np.float32(448.0)


def amax(x) -> np.float32:
    """max |x| over every element of a float32 array of bf16 values (0 if empty)."""
    x = np.asarray(x, dtype=np.float32)
    if x.size == 0:
        return np.float32(0.0)
    return np.float32(np.max(np.abs(x)))


def scales_from_amax(amax_eff) -> tuple:
    """Effective amax (float32 array) -> (descale, inv), both float32 arrays."""
    a = np.maximum(np.asarray(amax_eff, dtype=np.float32), AMAX_FLOOR)
    descale = (a / _FP8_MAX32).astype(np.float32)
    inv = (_FP8_MAX32 / a).astype(np.float32)
    return descale, inv


def static_amax_eff(static_amax, margin) -> np.ndarray:
    """Loaded amax values times the margin, one float32 multiply each."""
    return (np.asarray(static_amax, dtype=np.float32) * np.float32(margin)).astype(np.float32)


@dataclass
class ScaleState:
    """Scale state of one attention layer for tensors (Q, K, V).

    ``ring[t]`` holds the last ``history_len`` observed amax values of tensor
    ``t``; ``cursor`` counts dynamic forwards and selects the slot to
    overwrite.
    """

    history_len: int = HISTORY_LEN
    static_amax: object = None
    margin: float = 1.5
    ring: np.ndarray = field(default=None)
    cursor: int = 0
    amax_eff: np.ndarray = field(default=None)
    descale: np.ndarray = field(default=None)
    inv: np.ndarray = field(default=None)

    def __post_init__(self):
        if not 1 <= self.history_len <= HISTORY_LEN:
            raise ValueError("history_len must be in 1..16")
        self.ring = np.zeros((3, self.history_len), dtype=np.float32)
        self.amax_eff = np.zeros(3, dtype=np.float32)
        self.descale, self.inv = scales_from_amax(self.amax_eff)
        if self.static_amax is not None:
            sa = np.asarray(self.static_amax, dtype=np.float32)
            if sa.shape != (3,) or not np.all(np.isfinite(sa)) or np.any(sa <= 0):
                raise ValueError("static amax must be three finite positive values")
            m = np.float32(self.margin)
            if not np.isfinite(m) or m <= 0:
                raise ValueError("margin must be finite and positive")
            with np.errstate(over="ignore"):
                if not np.all(np.isfinite(static_amax_eff(sa, m))):
                    raise ValueError("static amax times margin overflows float32")
            self.static_amax = sa

    def forward_dynamic(self, observed) -> tuple:
        """Record this forward's observed amax of Q, K, V and return (descale, inv)."""
        observed = np.asarray(observed, dtype=np.float32)
        slot = self.cursor % self.history_len
        self.ring[:, slot] = observed
        self.cursor += 1
        self.amax_eff = self.ring.max(axis=1).astype(np.float32)
        self.descale, self.inv = scales_from_amax(self.amax_eff)
        return self.descale.copy(), self.inv.copy()

    def export_static_amax(self, margin=1.5) -> np.ndarray:
        """Calibrated amax to save: max over the ring of each tensor times the save margin (float32)."""
        if self.cursor == 0:
            raise ValueError("no dynamic forward has been observed")
        m = np.float32(margin)
        if not np.isfinite(m) or m <= 0:
            raise ValueError("margin must be finite and positive")
        ring_max = self.ring.max(axis=1).astype(np.float32)
        if np.any(ring_max <= 0):
            raise ValueError("a tensor observed only zeros")
        with np.errstate(over="ignore"):
            out = (ring_max * m).astype(np.float32)
        if not np.all(np.isfinite(out)):
            raise ValueError("amax times margin overflows float32")
        return out

    def forward_static(self) -> tuple:
        """Static mode: loaded amax times margin; observed values are ignored."""
        if self.static_amax is None:
            raise ValueError("static mode needs loaded scales")
        self.amax_eff = static_amax_eff(self.static_amax, self.margin)
        self.descale, self.inv = scales_from_amax(self.amax_eff)
        return self.descale.copy(), self.inv.copy()
