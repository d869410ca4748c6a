"""Scale-file I/O (host side, no GPU): the pages' format, aliases, refusals, exact round trip.

Pages: "FP8 ViT Encoder Attention", Scale File Format, and "FP8 vision
encoder attention", Create static scales: one object per vision attention
layer with numbers ``q``, ``k``, ``v``; ``q_scale``/``k_scale``/``v_scale``
are accepted as aliases.  The example the pages print is
``tests/golden/scale_file_example.json`` (its ``scales`` object).
"""

import json
import os

import numpy as np
import pytest

from quantized_flash_attn_amd import scale_file as sf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "scale_file_example.json")


def _write(tmp_path, obj, name="s.json"):
    p = tmp_path / name
    p.write_text(json.dumps(obj))
    return str(p)


def test_pages_example_loads(tmp_path):
    page = json.load(open(GOLDEN))["scales"]
    got = sf.load_scale_file(_write(tmp_path, page))
    assert got == {"visual.blocks.0.attn.attn": (224.0, 198.0, 210.0),
                   "visual.blocks.1.attn.attn": (218.0, 195.0, 207.0)}


def test_aliases(tmp_path):
    obj = {"visual.blocks.0.attn.attn": {"q_scale": 224.0, "k_scale": 198.0, "v_scale": 210.0},
           "visual.blocks.1.attn.attn": {"q": 218.0, "k_scale": 195.0, "v": 207, "v_scale": 207.0}}
    got = sf.load_scale_file(_write(tmp_path, obj))
    assert got["visual.blocks.0.attn.attn"] == (224.0, 198.0, 210.0)
    assert got["visual.blocks.1.attn.attn"] == (218.0, 195.0, 207.0)


@pytest.mark.parametrize("obj", [
    {},
    [],
    {"layer": {"q": 1.0, "k": 1.0}},                          # no v
    {"layer": {"q": 1.0, "k": 1.0, "v": 0.0}},                # not positive
    {"layer": {"q": 1.0, "k": -2.0, "v": 1.0}},
    {"layer": {"q": 1.0, "k": 1.0, "v": "3"}},                # not a number
    {"layer": {"q": True, "k": 1.0, "v": 1.0}},
    {"layer": {"q": 1.0, "k": 1.0, "v": 1e39}},               # overflows float32
    {"layer": {"q": 1.0, "q_scale": 2.0, "k": 1.0, "v": 1.0}},  # alias disagrees
    {"layer": [1.0, 1.0, 1.0]},
])
def test_refusals(tmp_path, obj):
    with pytest.raises(ValueError):
        sf.load_scale_file(_write(tmp_path, obj))


def test_nan_refused(tmp_path):
    p = tmp_path / "nan.json"
    p.write_text('{"layer": {"q": NaN, "k": 1.0, "v": 1.0}}')
    with pytest.raises(ValueError):
        sf.load_scale_file(str(p))


def test_round_trip_is_bit_exact(tmp_path):
    rng = np.random.default_rng(5)
    vals = (rng.uniform(0.5, 2.0, (40, 3)) * 2.0 ** rng.integers(-126, 120, (40, 3))).astype(np.float32)
    vals[0] = np.array([np.float32(1) / np.float32(3), np.float32(2.0 ** -149), np.finfo(np.float32).max], np.float32)
    scales = {f"visual.blocks.{i}.attn.attn": tuple(float(x) for x in vals[i]) for i in range(len(vals))}
    p = str(tmp_path / "rt.json")
    sf.save_scale_file(p, scales)
    raw = json.load(open(p))
    assert list(raw) == list(scales)
    assert all(set(v) == {"q", "k", "v"} for v in raw.values())
    got = sf.load_scale_file(p)
    for layer, want in scales.items():
        assert np.array_equal(np.array(got[layer], np.float32).view(np.uint32),
                              np.array(want, np.float32).view(np.uint32)), layer


def test_save_refuses_bad_values(tmp_path):
    for bad in ((1.0, 2.0), (1.0, 0.0, 1.0), (1.0, float("inf"), 1.0)):
        with pytest.raises(ValueError):
            sf.save_scale_file(str(tmp_path / "b.json"), {"layer": bad})
