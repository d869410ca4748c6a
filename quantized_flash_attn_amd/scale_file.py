"""Scale files: calibrate once with dynamic scaling, then load static scales.

Pages (cited by title and section):

* "FP8 ViT Encoder Attention", Calibrate-Once, Reuse Workflow, and "FP8
  vision encoder attention", Create static scales: run dynamic scaling over
  representative inputs, then write the learned per-layer scales, multiplied
  by a save margin (default 1.5), to a JSON file that later runs load as
  static scales.  The file is written after 16 forwards.
* Same pages, Scale File Format: one JSON object per vision attention layer,
  keyed by the layer name (e.g. ``visual.blocks.0.attn.attn``), holding the
  numbers ``q``, ``k`` and ``v``; ``q_scale``, ``k_scale`` and ``v_scale``
  are accepted in their place.

A stored value is an amax (range) value that already includes the margin, so
a state is initialised from it with margin 1.0.  Values are written as the
exact decimal of their float32 value, so a save/load round trip is
bit-exact.  This module is host-side I/O; the numbers come from the library
(``export_static_amax``) and go back into it (``init_scale_state``).
"""

import json
import math

import numpy as np

from . import export_static_amax, init_scale_state, read_scale_state

KEYS = ("q", "k", "v")
ALIASES = {"q": "q_scale", "k": "k_scale", "v": "v_scale"}
CALIBRATION_FORWARDS = 16


def _f32(x) -> float:
    return float(np.float32(x))


def _entry(layer: str, obj) -> tuple:
    if not isinstance(obj, dict):
        raise ValueError(f"scale file: entry {layer!r} is not an object")
    vals = []
    for key in KEYS:
        present = [k for k in (key, ALIASES[key]) if k in obj]
        if not present:
            raise ValueError(f"scale file: entry {layer!r} has no {key!r} (or {ALIASES[key]!r})")
        got = [obj[k] for k in present]
        for g in got:
            if isinstance(g, bool) or not isinstance(g, (int, float)):
                raise ValueError(f"scale file: {layer!r}.{key} is not a number")
        if len(got) == 2 and _f32(got[0]) != _f32(got[1]):
            raise ValueError(f"scale file: {layer!r} gives {key!r} and {ALIASES[key]!r} different values")
        v = _f32(got[0])
        if not math.isfinite(v) or not v > 0.0:
            raise ValueError(f"scale file: {layer!r}.{key} = {got[0]!r} must be finite and positive in float32")
        vals.append(v)
    return tuple(vals)


def load_scale_file(path) -> dict:
    """``{layer name: (q, k, v)}`` of float32 amax values from a scale file."""
    with open(path) as f:
        data = json.load(f)
    if not isinstance(data, dict) or not data:
        raise ValueError("scale file: expected a non-empty JSON object of layers")
    return {str(layer): _entry(str(layer), obj) for layer, obj in data.items()}


def save_scale_file(path, scales: dict) -> None:
    """Write ``{layer name: (q, k, v)}`` (margin already applied) in the pages' format."""
    out = {}
    for layer, vals in scales.items():
        vals = [_f32(x) for x in vals]
        if len(vals) != 3 or not all(math.isfinite(v) and v > 0.0 for v in vals):
            raise ValueError(f"scale file: {layer!r} needs three finite positive values")
        out[str(layer)] = dict(zip(KEYS, vals))
    with open(path, "w") as f:
        json.dump(out, f, indent=2)
        f.write("\n")


def calibrated_scales(states: dict, margin: float = 1.5, min_forwards: int = CALIBRATION_FORWARDS) -> dict:
    """``{layer: (q, k, v)}`` learned by dynamic forwards on each layer's state.

    Each value is fp32(ring maximum * margin).  A layer whose state has seen
    fewer than ``min_forwards`` dynamic forwards is refused: the pages write
    the file after 16 forwards, when the 16-entry ring is full.
    """
    out = {}
    for layer, st in states.items():
        seen = read_scale_state(st)["cursor"]
        if seen < min_forwards:
            raise ValueError(f"layer {layer!r} has seen {seen} dynamic forwards, fewer than {min_forwards}")
        out[str(layer)] = tuple(export_static_amax(st, margin))
    return out


def calibrate_to_file(path, states: dict, margin: float = 1.5, min_forwards: int = CALIBRATION_FORWARDS) -> dict:
    """Export every layer's calibrated scales and write the scale file; returns what was written."""
    scales = calibrated_scales(states, margin, min_forwards)
    save_scale_file(path, scales)
    return scales


def init_scale_state_from_file(path, layer: str, device=None, history_len: int = CALIBRATION_FORWARDS, buffer=None):
    """A scale state for ``layer`` with the file's static amax values (margin 1.0)."""
    scales = load_scale_file(path)
    if layer not in scales:
        raise KeyError(f"scale file has no layer {layer!r}")
    return init_scale_state(device=device, history_len=history_len, static_amax=scales[layer], margin=1.0,
                            buffer=buffer)
