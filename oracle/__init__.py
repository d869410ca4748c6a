"""CPU oracle for FP8 ViT encoder attention -- TEST INFRASTRUCTURE ONLY.

This package is the slow, plain definition that the HIP library is checked
against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import it.  The library under
``quantized_flash_attn_amd/`` never imports, links or calls anything here, and
nothing here imports the library: the two share no code.  The only module both
sides use is ``workloads.py`` (seeded synthetic inputs, none of the method's
arithmetic).

What it computes, and where the pages say so (pages are cited by title and
section):

* ``e4m3``     -- the OCP FP8 E4M3 ("fn") codec.  The pages only say "FP8"
                  ("FP8 ViT Encoder Attention", intro; "FP8 vision encoder
                  attention", Requirements); the format is a reading of them.
* ``scales``   -- per-tensor amax, the 16-entry circular buffer of observed
                  amax values that sets per-forward scales ("FP8 ViT Encoder
                  Attention", Usage; "FP8 vision encoder attention", Enable FP8
                  attention), and static scales times a save margin of 1.5
                  ("FP8 ViT Encoder Attention", Calibrate-Once, Reuse Workflow;
                  "FP8 vision encoder attention", Create static scales).
* ``quantize`` -- on-the-fly quantization of Q, K and V to FP8 before the
                  attention call ("FP8 ViT Encoder Attention", intro).
* ``attention``-- softmax attention over packed variable-length sequences with
                  per-tensor scales ("FP8 vision encoder attention",
                  Requirements: packed variable-length batches, a per-tensor
                  FP8 varlen attention function), in float64; the same
                  definition on bf16 inputs for the BF16 baseline ("FP8 ViT
                  Encoder Attention", Performance).

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
something other than itself (the OCP format table, torch-CPU's float8 cast,
closed forms, IEEE identities, brute force, torch-CPU fp64 SDPA and
invariants).  No function is "parity unpinned".
"""

from .e4m3 import DECODE_TABLE, decode, encode, FP8_MAX
from .scales import (
    AMAX_FLOOR,
    HISTORY_LEN,
    ScaleState,
    amax,
    scales_from_amax,
    static_amax_eff,
)
from .quantize import quantize, quantize_qkv, quantize_qkv_packed
from .attention import attention, attention_float, attention_float_rows, attention_rows

__all__ = [
    "DECODE_TABLE",
    "decode",
    "encode",
    "FP8_MAX",
    "AMAX_FLOOR",
    "HISTORY_LEN",
    "ScaleState",
    "amax",
    "scales_from_amax",
    "static_amax_eff",
    "quantize",
    "quantize_qkv",
    "quantize_qkv_packed",
    "attention",
    "attention_rows",
    "attention_float",
    "attention_float_rows",
]
