"""C ABI checks that need no GPU: exported symbols and argument validation.

Every entry point validates its arguments on the host before any HIP call,
so each error status here is reached without touching a device.  The fake
device pointers are never dereferenced.
"""

import ctypes
import os
import re
import subprocess

import pytest

import quantized_flash_attn_amd as qfa

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "qfa.h")
lib = qfa.raw_library()
FAKE = 0x10000          # 16-byte aligned, never dereferenced
MISALIGNED = 0x10004

OK, NULL, SHAPE, UNSUP, ALIGN, MODE, NO_STATIC, VALUE, STATE = 0, 1, 2, 3, 4, 5, 6, 7, 8
WORKSPACE = 11


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qfa_[a-z_0-9]+)\s*\(", text)))


def test_header_symbols_exported():
    declared = header_functions()
    assert len(declared) == 17, declared
    out = subprocess.run(["nm", "-D", "--defined-only", qfa.library_path()], stdout=subprocess.PIPE, text=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    missing = [f for f in declared if f not in exported]
    assert not missing, missing
    assert set(declared) == set(qfa.EXPORTS)


def test_state_bytes_and_status_strings():
    assert 256 <= qfa.scale_state_bytes() <= 64 * 1024
    for s in range(12):
        assert lib.qfa_status_string(s) != b"unknown status", s
    assert lib.qfa_status_string(99) == b"unknown status"


def _init(handle, buf=FAKE, hist=16, static=None, margin=1.5):
    sa = None if static is None else (ctypes.c_float * 3)(*static)
    return lib.qfa_init_scale_state(handle, buf, hist, sa, ctypes.c_float(margin), None)


def test_init_validation():
    h = qfa._State()
    assert _init(None) == NULL
    assert _init(ctypes.byref(h), buf=None) == NULL
    assert _init(ctypes.byref(h), buf=MISALIGNED) == ALIGN
    for hist in (0, 17, -3):
        assert _init(ctypes.byref(h), hist=hist) == VALUE
    for bad in ([1.0, 0.0, 1.0], [1.0, -2.0, 3.0], [float("nan"), 1.0, 1.0], [float("inf"), 1.0, 1.0]):
        assert _init(ctypes.byref(h), static=bad) == VALUE
    assert _init(ctypes.byref(h), static=[3e38, 1.0, 1.0], margin=1.5) == VALUE   # product overflows
    for m in (0.0, -1.5, float("inf"), float("nan")):
        assert _init(ctypes.byref(h), static=[1.0, 1.0, 1.0], margin=m) == VALUE
    assert h.magic == 0                      # nothing was initialised
    assert b"history_len" in lib.qfa_last_error() or lib.qfa_last_error()


def _handle(has_static=0, magic=0x31414651):
    h = qfa._State()
    h.magic = magic
    h.history_len = 16
    h.has_static = has_static
    h.device = FAKE
    return h


def _quant(h, mode=0, ptrs=(FAKE,) * 6, T=8, H=2, D=128):
    q, k, v, q8, k8, v8 = ptrs
    return lib.qfa_quantize_qkv(h, mode, q, k, v, T, H, D, q8, k8, v8, None)


def test_quantize_validation():
    assert _quant(None) == NULL
    assert _quant(ctypes.byref(_handle(magic=0))) == STATE
    h = _handle()
    assert _quant(ctypes.byref(h), mode=2) == MODE
    assert _quant(ctypes.byref(h), mode=-1) == MODE
    assert _quant(ctypes.byref(h), mode=1) == NO_STATIC
    assert _quant(ctypes.byref(h), D=64) == UNSUP
    assert _quant(ctypes.byref(h), H=0) == SHAPE
    assert _quant(ctypes.byref(h), T=-1) == SHAPE
    assert _quant(ctypes.byref(h), T=1 << 40) == SHAPE
    for i in range(6):
        p = [FAKE] * 6
        p[i] = None
        assert _quant(ctypes.byref(h), ptrs=tuple(p)) == NULL
        p[i] = MISALIGNED
        assert _quant(ctypes.byref(h), ptrs=tuple(p)) == ALIGN
    hs = _handle(has_static=1)
    assert _quant(ctypes.byref(hs), mode=1, D=100) == UNSUP


@pytest.mark.parametrize("entry", ["qfa_fp8_varlen_attn", "qfa_fp8_varlen_attn_fp8qk"])
def test_attention_validation(entry):
    fn = getattr(lib, entry)

    def _attn(q8=FAKE, k8=FAKE, v8=FAKE, sc=FAKE, cu=FAKE, B=1, T=8, H=2, D=128, out=FAKE):
        return fn(q8, k8, v8, sc, cu, B, T, H, D, out, None)

    for d in (0, 4, 100, 136, 256):
        assert _attn(D=d) == UNSUP, d
    assert _attn(H=0) == SHAPE
    assert _attn(T=-5) == SHAPE
    assert _attn(B=0) == SHAPE
    assert _attn(T=1 << 31, H=1) == SHAPE
    assert _attn(T=1, H=65537) == SHAPE     # the tile loads' 32-bit descriptor range bounds the head count
    assert _attn(sc=None) == NULL
    assert _attn(cu=None) == NULL
    for name in ("q8", "k8", "v8", "out"):
        assert _attn(**{name: None}) == NULL
        assert _attn(**{name: MISALIGNED}) == ALIGN
    assert _attn(sc=FAKE + 2) == ALIGN
    assert _attn(cu=FAKE + 1) == ALIGN
    # sequence count and grid: (T/256 + B) query tiles per head, times the heads, must fit an int
    assert _attn(B=(1 << 30) + 1) == SHAPE
    assert _attn(B=2 ** 31 - 1, T=(1 << 31) - 1) == SHAPE
    assert _attn(B=1 << 30, T=8, H=4) == SHAPE
    assert b"grid" in lib.qfa_last_error()


def _split(q8=FAKE, k8=FAKE, v8=FAKE, sc=FAKE, cu=FAKE, B=1, T=300, H=2, D=128, S=0, ws=FAKE, wsb=1 << 30,
           out=FAKE):
    return lib.qfa_fp8_varlen_attn_split(q8, k8, v8, sc, cu, B, T, H, D, S, ws, wsb, out, None)


def test_split_attention_validation():
    # the checks shared with qfa_fp8_varlen_attn
    assert _split(D=100) == UNSUP
    assert _split(H=0) == SHAPE
    assert _split(B=0) == SHAPE
    assert _split(T=1, H=65537) == SHAPE
    assert _split(sc=None) == NULL
    for name in ("q8", "k8", "v8", "out"):
        assert _split(**{name: None}) == NULL
        assert _split(**{name: MISALIGNED}) == ALIGN
    # split count and workspace
    for bad in (-1, 17, 100):
        assert _split(S=bad) == VALUE, bad
    need = lib.qfa_fp8_varlen_attn_workspace_bytes(1, 300, 2, 4)
    assert need > 0
    assert _split(S=4, ws=None) == WORKSPACE
    assert _split(S=4, wsb=need - 1) == WORKSPACE
    assert _split(S=4, ws=MISALIGNED, wsb=need) == ALIGN
    # the automatic count for 2304 tokens x 8 heads is above 1, so a workspace is required
    assert lib.qfa_fp8_varlen_attn_auto_splits(1, 2304, 8) > 1
    assert _split(S=0, ws=None, T=2304, H=8) == WORKSPACE
    # ... and for 300 tokens x 2 heads it is 1: no workspace needed (validation passes; nothing to launch
    # here would need a GPU, so only the count is checked)
    assert lib.qfa_fp8_varlen_attn_auto_splits(1, 300, 2) == 1
    assert b"workspace" in lib.qfa_last_error()
    # 16 ranges, or 16 merge workgroups per query tile, past the grid limit
    assert _split(B=1 << 26, T=8, H=2, S=16, wsb=2 ** 62) == SHAPE
    assert _split(B=1 << 26, T=8, H=2, S=2, wsb=2 ** 62) == SHAPE
    assert b"grid" in lib.qfa_last_error()


def test_noalloc_split_validation():
    def na(B=1, T=2304, H=8, D=128, S=0, out=FAKE, sc=FAKE):
        return lib.qfa_fp8_varlen_attn_split_noalloc(FAKE, FAKE, FAKE, sc, FAKE, B, T, H, D, S, out, None)
    assert na(D=100) == UNSUP
    assert na(sc=None) == NULL
    assert na(out=MISALIGNED) == ALIGN
    assert na(S=17) == VALUE and na(S=-1) == VALUE
    # requests beyond the library's fixed workspace are refused before anything is enqueued
    assert lib.qfa_fp8_varlen_attn_workspace_bytes(1, 99504, 16, 16) > qfa.NOALLOC_SCRATCH_BYTES
    assert na(T=99504, H=16, S=16) == WORKSPACE
    assert b"workspace" in lib.qfa_last_error()
    # every automatic split count fits it (at most 512 virtual query tiles x 256 rows of 264 bytes)
    assert 512 * 256 * 264 <= qfa.NOALLOC_SCRATCH_BYTES
    for B, T, H in ((1, 2304, 8), (1, 8192, 4), (1, 4096, 1), (1, 2304, 1), (3, 700, 5), (1, 60000, 2)):
        assert lib.qfa_fp8_varlen_attn_workspace_bytes(B, T, H, 0) <= qfa.NOALLOC_SCRATCH_BYTES, (B, T, H)


def test_split_counts_and_workspace_sizes():
    auto = lib.qfa_fp8_varlen_attn_auto_splits
    wsb = lib.qfa_fp8_varlen_attn_workspace_bytes
    # launches with a query tile per CU are not split
    assert auto(1, 8192, 16) == 1 and wsb(1, 8192, 16, 0) == 0
    assert auto(1, 8192, 8) == 1           # exactly 256 query tiles
    assert auto(3, 43200, 16) == 1 and auto(4, 99504, 16) == 1
    # as many ranges as fit one round of 256 workgroups, each of at least two key tiles
    assert auto(1, 2304, 16) == 1          # 144 query tiles: two ranges would need a second round
    assert auto(1, 2304, 8) == 3           # 72 query tiles x 3 ranges = 216
    assert auto(1, 8192, 4) == 2           # 128 x 2 = 256
    assert auto(1, 4096, 1) == 16          # 16 x 16, two key tiles per range
    assert auto(1, 256, 2) == 1            # two key tiles: one range of two
    assert auto(1, 1, 1) == 1
    # bytes: S ranges x heads x virtual tiles (T/256 + B) x 256 rows x (128 fp16 + 2 float32)
    for B, T, H, S in ((1, 2304, 16, 3), (4, 1000, 3, 5), (2, 257, 1, 16), (1, 2304, 8, 3)):
        rows = S * H * (T // 256 + B) * 256
        o = (rows * 256 + 255) // 256 * 256
        assert wsb(B, T, H, S) == o + rows * 8, (B, T, H, S)
    assert wsb(1, 2304, 16, 1) == 0 and wsb(1, 2304, 16, 0) == 0
    assert wsb(1, 2304, 8, 0) == wsb(1, 2304, 8, 3)
    assert wsb(1, 2304, 16, 17) == 0 and wsb(0, 2304, 16, 2) == 0 and wsb(1, -1, 16, 2) == 0
    # out-of-range sizes: no count above 1, no workspace, no overflow
    assert auto(1, 2 ** 63 - 1, 16) == 1 and auto(2 ** 31 - 1, 1000, 1) == 1 and auto(1, 1 << 31, 1) == 1
    assert wsb(1, 1 << 31, 1, 2) == 0 and wsb((1 << 30) + 1, 8, 1, 2) == 0 and wsb(1, 2304, 65537, 2) == 0


def _packed(h, mode=0, qkv=FAKE, T=8, H=2, D=80, outs=(FAKE,) * 3):
    return lib.qfa_quantize_qkv_packed(h, mode, qkv, T, H, D, outs[0], outs[1], outs[2], None)


def test_packed_quantize_validation():
    assert _packed(None) == NULL
    assert _packed(ctypes.byref(_handle(magic=0))) == STATE
    h = _handle()
    assert _packed(ctypes.byref(h), mode=3) == MODE
    assert _packed(ctypes.byref(h), mode=1) == NO_STATIC
    for d in (0, 4, 12, 100, 136):
        assert _packed(ctypes.byref(h), D=d) == UNSUP, d
    assert _packed(ctypes.byref(h), H=0) == SHAPE
    assert _packed(ctypes.byref(h), T=-1) == SHAPE
    assert _packed(ctypes.byref(h), T=1 << 27, H=1) == SHAPE          # 16 output chunks per row exceed 2^31
    assert _packed(ctypes.byref(h), qkv=None) == NULL
    assert _packed(ctypes.byref(h), qkv=MISALIGNED) == ALIGN
    for i in range(3):
        o = [FAKE] * 3
        o[i] = None
        assert _packed(ctypes.byref(h), outs=tuple(o)) == NULL
        o[i] = MISALIGNED
        assert _packed(ctypes.byref(h), outs=tuple(o)) == ALIGN


def _battn(q=FAKE, k=FAKE, v=FAKE, cu=FAKE, B=1, T=8, H=2, D=128, out=FAKE):
    return lib.qfa_bf16_varlen_attn(q, k, v, cu, B, T, H, D, out, None)


def test_bf16_attention_validation():
    assert _battn(D=64) == UNSUP
    assert _battn(H=0) == SHAPE
    assert _battn(T=-5) == SHAPE
    assert _battn(B=0) == SHAPE
    assert _battn(T=1 << 31, H=1) == SHAPE
    assert _battn(T=1, H=65537) == SHAPE
    assert _battn(cu=None) == NULL
    for name in ("q", "k", "v", "out"):
        assert _battn(**{name: None}) == NULL
        assert _battn(**{name: MISALIGNED}) == ALIGN
    assert _battn(cu=FAKE + 1) == ALIGN


def test_other_entry_points_validation():
    assert lib.qfa_descale_ptr(None) is None
    assert lib.qfa_descale_ptr(ctypes.byref(_handle(magic=0))) is None
    assert lib.qfa_read_scale_state(None, None, None) == NULL
    snap = qfa._Snapshot()
    assert lib.qfa_read_scale_state(ctypes.byref(_handle(magic=0)), ctypes.byref(snap), None) == STATE
    assert lib.qfa_check_cu_seqlens(None, 1, 8, None) == NULL
    assert lib.qfa_check_cu_seqlens(FAKE, 0, 8, None) == SHAPE
    assert lib.qfa_check_cu_seqlens(FAKE, 1, -1, None) == SHAPE
    out = (ctypes.c_float * 3)()
    assert lib.qfa_export_static_amax(None, 1.5, out, None) == NULL
    assert lib.qfa_export_static_amax(ctypes.byref(_handle()), 1.5, None, None) == NULL
    assert lib.qfa_export_static_amax(ctypes.byref(_handle(magic=0)), 1.5, out, None) == STATE
    for m in (0.0, -1.5, float("inf"), float("nan")):
        assert lib.qfa_export_static_amax(ctypes.byref(_handle()), m, out, None) == VALUE


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros((4, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        qfa.quantize_qkv(None, "dynamic", x, x, x)
    c = torch.zeros((4, 2, 128), dtype=torch.uint8)
    with pytest.raises(ValueError):
        qfa.fp8_varlen_attn(c, c, c, torch.ones(3), torch.tensor([0, 4], dtype=torch.int32), 2)
