"""Host-side tests of the C ABI (no GPU): the library loads, exports every
function include/fp4q.h declares, and rejects every invalid configuration
with its documented status before anything is enqueued (no compute call is
made: every call here either fails validation or has an empty tensor).

The calls pass placeholder device addresses; a call that validated would
launch on them, so where a GPU is visible these tests do not run (without
one such a launch fails with FP4Q_ERR_HIP, which every helper rejects)."""
import ctypes as ct
import os
import re

import pytest
import torch

import block_scaled_fp4_amax_amd as fq

pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                reason="placeholder device pointers: host-only validation tests")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4q.h")

FAKE = 0x10000       # 16-byte aligned, never dereferenced: validation fails first
FAKE_MIS = 0x10004   # 4-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp4q?_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"fp4_quantize", "fp4_dequantize", "fp4_qdq", "fp4_cast_transpose", "fp4_cast_transpose_grouped",
            "fp4q_abi_version", "fp4q_status_str", "fp4q_buffer_sizes", "fp4q_workspace_bytes"} <= set(names)
    L = ct.CDLL(fq.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert fq.fp4q_abi_version() == fq.ABI_VERSION


def test_status_strings():
    for st in range(10):
        assert fq.fp4q_status_str(st)
    assert fq.fp4q_status_str(123) == "unknown status"


def _validated(st):
    assert st != fq.ERR_HIP, "a call reached a launch"
    return st


def q(cfg, rows=64, cols=64, ld=None, x=FAKE, codes=FAKE, scales=FAKE, outer=FAKE, residual=None, ws=None, wsb=0):
    return _validated(fq.lib().fp4_quantize(ct.byref(cfg), x, rows, cols, cols if ld is None else ld, codes, scales,
                                            outer, residual, ws, wsb, None))


def qdq(cfg, rows=64, cols=64, ld=None, x=FAKE, y=FAKE):
    return _validated(fq.lib().fp4_qdq(ct.byref(cfg), x, rows, cols, cols if ld is None else ld, y, None, None, None,
                                       None, None, 0, None))


def ct_(cfg, rows=64, cols=64, ld=None, x=FAKE, row_outer=FAKE, col_outer=None, residual=None, ws=None, wsb=0,
        col_codes=FAKE):
    return _validated(fq.lib().fp4_cast_transpose(ct.byref(cfg), x, rows, cols, cols if ld is None else ld, FAKE, FAKE,
                                                  row_outer, col_codes, FAKE, col_outer, residual, ws, wsb, None))


def test_mode_rules():
    C = fq.make_cfg
    # two_level_scaling is one of none / tensorwise / outer_block; outer knobs only in outer-block mode
    assert q(C(two_level="tensorwise", outer_block_size=64)) == fq.ERR_MODE
    assert q(C(two_level="none", outer_2d=True)) == fq.ERR_MODE
    assert q(C(two_level=7)) == fq.ERR_MODE
    # outer_block_size: a multiple of 16 that divides the reduction dims
    assert q(C(two_level="outer_block", outer_block_size=24)) == fq.ERR_SHAPE
    assert q(C(two_level="outer_block", outer_block_size=0)) == fq.ERR_SHAPE
    assert q(C(two_level="outer_block", outer_block_size=64), cols=2880 - 2880 % 64 + 32, ld=None) == fq.ERR_SHAPE
    assert q(C(two_level="outer_block", outer_block_size=128), cols=2880) == fq.ERR_SHAPE   # 2880 % 128 != 0
    # scale-format pins: AMD-FP4 is UE5M3; MXFP4 is UE8M0; NVFP4 may use E4M3 or UE5M3
    assert q(C(format="amdfp4", scale_format="e4m3")) == fq.ERR_MODE
    assert q(C(format="mxfp4", scale_format="e4m3")) == fq.ERR_MODE
    assert q(C(format="nvfp4", scale_format="ue8m0")) == fq.ERR_MODE
    assert q(C(format="mxfp4", two_level="tensorwise")) == fq.ERR_MODE
    assert q(C(format="mxfp4", rounding="stochastic")) == fq.ERR_UNSUPPORTED
    assert q(C(format=9)) == fq.ERR_MODE
    # precomputed outer without a two-level mode
    assert q(C(outer_mode=1)) == fq.ERR_MODE
    # dtype guard: fp16 rejected as input and as output ("MXFP4 weight QAT
    # recipes", Guards); fp32 accepted by the rowwise paths only
    assert q(C(input_dtype="fp16")) == fq.ERR_DTYPE
    assert q(C(input_dtype=7)) == fq.ERR_DTYPE
    assert qdq(C(output_dtype="fp16")) == fq.ERR_DTYPE
    assert qdq(C(format="mxfp4", output_dtype=5)) == fq.ERR_DTYPE
    for f32 in (C(input_dtype="fp32"), C(format="mxfp4", input_dtype="fp32", output_dtype="fp32")):
        assert q(f32, rows=0, x=None, codes=None, scales=None, outer=None) == fq.OK
    tile2d = dict(two_level="outer_block", outer_block_size=64, outer_2d=True)
    assert q(C(input_dtype="fp32", **tile2d)) == fq.ERR_UNSUPPORTED
    assert q(C(input_dtype="fp32", inner_2d=True)) == fq.ERR_UNSUPPORTED
    assert qdq(C(output_dtype="fp32", **tile2d)) == fq.ERR_UNSUPPORTED
    assert ct_(C(input_dtype="fp32")) == fq.ERR_UNSUPPORTED
    bad = C()
    bad.abi_version = 99
    assert q(bad) == fq.ERR_ABI
    assert fq.lib().fp4_quantize(None, FAKE, 1, 16, 16, FAKE, FAKE, None, None, None, 0, None) == fq.ERR_NULL


def test_shape_and_pointer_rules():
    C = fq.make_cfg
    assert q(C(), cols=40) == fq.ERR_SHAPE                      # cols % 16
    assert q(C(format="mxfp4"), cols=48) == fq.ERR_SHAPE        # cols % 32
    assert q(C(), rows=-1) == fq.ERR_SHAPE
    assert q(C(), cols=64, ld=32) == fq.ERR_SHAPE               # ld < cols
    # any row pitch for the rowwise paths (views), 16-byte rows for the tile kernels
    assert q(C(), rows=0, cols=64, ld=68, x=None, codes=None, scales=None, outer=None) == fq.OK
    tile2d = C(two_level="outer_block", outer_block_size=64, outer_2d=True)
    assert q(tile2d, cols=64, ld=68) == fq.ERR_ALIGN
    assert ct_(C(), cols=64, ld=68) == fq.ERR_ALIGN
    assert q(C(), x=None) == fq.ERR_NULL
    assert q(C(), codes=None) == fq.ERR_NULL
    assert q(C(two_level="tensorwise"), outer=None) == fq.ERR_NULL
    # misaligned views: x aligned to its element size is enough for the rowwise paths
    assert q(C(), x=FAKE + 1) == fq.ERR_ALIGN
    assert q(C(input_dtype="fp32"), x=FAKE + 2) == fq.ERR_ALIGN
    assert q(C(format="mxfp4", input_dtype="fp32"), x=FAKE + 6) == fq.ERR_ALIGN
    assert q(tile2d, x=FAKE_MIS) == fq.ERR_ALIGN
    assert ct_(C(), x=FAKE_MIS) == fq.ERR_ALIGN
    assert qdq(C(), y=FAKE_MIS) == fq.ERR_ALIGN                 # outputs stay 16-byte aligned
    assert q(C(format="mxfp4"), residual=FAKE) == fq.ERR_UNSUPPORTED
    # 2D outer needs rows % obs; only obs 64 is built for 2D
    assert q(C(two_level="outer_block", outer_block_size=64, outer_2d=True), rows=80) == fq.ERR_SHAPE
    assert q(C(two_level="outer_block", outer_block_size=32, outer_2d=True)) == fq.ERR_UNSUPPORTED
    # tensorwise needs a workspace of fp4q_workspace_bytes()
    cfg = C(two_level="tensorwise")
    need = fq.fp4q_workspace_bytes(cfg, 64, 64)
    assert need > 0
    assert q(cfg, ws=None, wsb=0) == fq.ERR_NULL
    assert q(cfg, ws=FAKE, wsb=need - 4) == fq.ERR_WORKSPACE


def test_cast_transpose_rules():
    C = fq.make_cfg
    assert ct_(C(), rows=40) == fq.ERR_SHAPE                    # rows % 16 for the columnwise buffer
    assert ct_(C(format="mxfp4")) == fq.ERR_UNSUPPORTED
    o1 = C(two_level="outer_block", outer_block_size=64)
    assert ct_(o1, col_outer=None) == fq.ERR_NULL               # 1D needs its columnwise outer array
    assert ct_(o1, rows=96, col_outer=FAKE) == fq.ERR_SHAPE     # rows % obs in 1D columnwise
    o2 = C(two_level="outer_block", outer_block_size=64, outer_2d=True)
    assert ct_(o2, col_outer=FAKE + 4096) == fq.ERR_MODE        # 2D outer is shared
    assert ct_(o2, col_codes=None) == fq.ERR_NULL
    # 1D groups of 128 are built (a pre-pass computes their scales); 256 is valid but not built
    assert ct_(C(two_level="outer_block", outer_block_size=128), rows=64, cols=128, col_outer=FAKE) == fq.ERR_SHAPE
    assert ct_(C(two_level="outer_block", outer_block_size=256), rows=256, cols=256, col_outer=FAKE) == fq.ERR_UNSUPPORTED


def test_grouped_rules():
    C = fq.make_cfg
    cfg = C(two_level="outer_block", outer_block_size=64, outer_2d=True)
    L = fq.lib()
    rows = (ct.c_int64 * 2)(64, 80)
    args = (64, FAKE, 64, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, 0, None)
    assert L.fp4_cast_transpose_grouped(ct.byref(cfg), 2, rows, *args) == fq.ERR_SHAPE
    assert L.fp4_cast_transpose_grouped(ct.byref(cfg), -1, rows, *args) == fq.ERR_SHAPE
    assert L.fp4_cast_transpose_grouped(ct.byref(cfg), 2, None, *args) == fq.ERR_NULL
    assert L.fp4_cast_transpose_grouped(ct.byref(C(two_level="tensorwise")), 1, rows, *args) == fq.ERR_UNSUPPORTED
    # zero groups is an empty call
    assert L.fp4_cast_transpose_grouped(ct.byref(cfg), 0, None, *args) == fq.OK


def test_inner_2d_rules():
    """16 x 16 inner tiles ("Block-Scaled FP8 and FP4 Weight Quantization",
    section 6): NVFP4 / AMD-FP4 only, not with 1D outer groups (each direction
    would be normalised differently), whole 16-row bands."""
    C = fq.make_cfg
    L = fq.lib()
    assert q(C(format="mxfp4", inner_2d=True)) == fq.ERR_MODE
    assert q(C(two_level="outer_block", outer_block_size=64, inner_2d=True)) == fq.ERR_MODE
    assert ct_(C(two_level="outer_block", outer_block_size=64, inner_2d=True), col_outer=FAKE) == fq.ERR_MODE
    bad = C()
    bad.inner_2d = 2
    assert q(bad) == fq.ERR_MODE
    assert q(C(inner_2d=True), rows=40) == fq.ERR_SHAPE          # rows % 16, also rowwise
    assert q(C(inner_2d=True), rows=40, cols=64) == fq.ERR_SHAPE
    y = fq.lib().fp4_qdq(ct.byref(C(inner_2d=True)), FAKE, 24, 64, 64, FAKE, None, None, None, None, None, 0, None)
    assert y == fq.ERR_SHAPE
    cfg = C(two_level="outer_block", outer_block_size=64, outer_2d=True, inner_2d=True)
    rows = (ct.c_int64 * 2)(64, 72)
    args = (64, FAKE, 64, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, 0, None)
    assert L.fp4_cast_transpose_grouped(ct.byref(cfg), 2, rows, *args) == fq.ERR_SHAPE
    # the sizes of a 16 x 16 layout are those of the 1 x 16 one (scales replicated per row)
    s = fq.fp4q_buffer_sizes(C(inner_2d=True, two_level="tensorwise"), 256, 512)
    assert s["row_scales"] == 256 * 32 and s["col_scales"] == 512 * 16
    with pytest.raises(fq.Fp4Error):
        fq.fp4q_buffer_sizes(C(inner_2d=True), 40, 64)
    # empty tensors validate the configuration only
    assert q(C(inner_2d=True), rows=0, x=None, codes=None, scales=None, outer=None) == fq.OK


def test_mx_project_fp8_rules():
    """The MXFP4 projection with FP8 re-encodings: MXFP4 only, 1x32 blocks,
    32x1 columnwise blocks and 128x128 blocks must tile the tensor."""
    C = fq.make_cfg
    L = fq.lib()

    def call(cfg, rows=128, cols=128, ld=None, x=FAKE, y=FAKE, r8=FAKE, r8s=FAKE, c8=FAKE, c8s=FAKE, b=FAKE,
             bt=FAKE, bs=FAKE):
        return _validated(L.fp4_mx_project_fp8(ct.byref(cfg), x, rows, cols, cols if ld is None else ld, y, r8, r8s,
                                               c8, c8s, b, bt, bs, None))
    mx = C(format="mxfp4")
    assert call(C()) == fq.ERR_MODE                                     # NVFP4 is not the projection
    assert call(C(format="mxfp4", rounding="stochastic")) == fq.ERR_UNSUPPORTED
    assert call(mx, cols=144) == fq.ERR_SHAPE                           # cols % 32
    assert call(mx, rows=48, b=None, bt=None, bs=None) == fq.ERR_SHAPE  # rows % 32 for the columnwise blocks
    assert call(mx, rows=96) == fq.ERR_SHAPE                            # rows % 128 for 128x128 blocks
    assert call(mx, r8s=None) == fq.ERR_NULL                            # payload without its scales
    assert call(mx, c8=None) == fq.ERR_NULL
    assert call(mx, x=None) == fq.ERR_NULL
    assert call(mx, x=FAKE_MIS) == fq.ERR_ALIGN
    assert call(mx, ld=132) == fq.ERR_ALIGN                              # 16-byte rows
    assert call(C(format="mxfp4", input_dtype="fp32")) == fq.ERR_UNSUPPORTED
    assert call(C(format="mxfp4", output_dtype="fp32")) == fq.ERR_UNSUPPORTED
    assert call(mx, rows=(1 << 22) + 128) == fq.ERR_UNSUPPORTED
    assert call(mx, rows=0, x=None) == fq.OK                            # empty: validated, nothing launched


def test_empty_tensors_are_accepted_without_launch():
    C = fq.make_cfg
    for cfg in (C(), C(format="mxfp4"), C(two_level="outer_block", outer_block_size=64, outer_2d=True)):
        assert q(cfg, rows=0, x=None, codes=None, scales=None, outer=None) == fq.OK
    assert fq.lib().fp4_dequantize(ct.byref(C()), None, None, None, 0, 16, 0, None, None) == fq.OK


def test_dequantize_rules():
    C = fq.make_cfg
    L = fq.lib()
    assert L.fp4_dequantize(ct.byref(C()), FAKE, FAKE, None, 16, 40, 0, FAKE, None) == fq.ERR_SHAPE
    assert L.fp4_dequantize(ct.byref(C()), FAKE, FAKE, None, 16, 32, 1, FAKE, None) == fq.ERR_MODE
    o2 = C(two_level="outer_block", outer_block_size=64, outer_2d=True)
    assert L.fp4_dequantize(ct.byref(o2), FAKE, FAKE, None, 64, 64, 0, FAKE, None) == fq.ERR_NULL
    assert L.fp4_dequantize(ct.byref(o2), FAKE, FAKE, FAKE, 48, 64, 0, FAKE, None) == fq.ERR_SHAPE
    assert L.fp4_dequantize(ct.byref(C(output_dtype="fp16")), FAKE, FAKE, None, 16, 32, 0, FAKE, None) == fq.ERR_DTYPE
    assert L.fp4_dequantize(ct.byref(C(output_dtype="fp32")), FAKE, FAKE, None, 16, 32, 0, FAKE_MIS,
                            None) == fq.ERR_ALIGN
    # buffer sizes follow the output dtype
    assert fq.fp4q_buffer_sizes(C(output_dtype="fp32"), 32, 64)["y"] == 32 * 64 * 4
    assert fq.fp4q_buffer_sizes(C(), 32, 64)["y"] == 32 * 64 * 2


def test_buffer_sizes():
    C = fq.make_cfg
    s = fq.fp4q_buffer_sizes(C(two_level="outer_block", outer_block_size=64), 16384, 2880)
    assert s["row_codes"] == 16384 * 1440 and s["row_scales"] == 16384 * 180
    assert s["row_outer"] == 16384 * 45 * 4 and s["col_outer"] == 2880 * 256 * 4
    assert s["col_codes"] == 2880 * 8192 and s["col_scales"] == 2880 * 1024
    s2 = fq.fp4q_buffer_sizes(C(two_level="outer_block", outer_block_size=64, outer_2d=True), 4096, 4096)
    assert s2["row_outer"] == 64 * 64 * 4 and s2["col_outer"] == 0
    s3 = fq.fp4q_buffer_sizes(C(format="mxfp4"), 8192, 8192)
    assert s3["row_scales"] == 8192 * 256 and s3["col_codes"] == 0 and s3["residual"] == 0
    assert fq.fp4q_buffer_sizes(C(two_level="tensorwise"), 256, 256)["workspace"] > 0
    with pytest.raises(fq.Fp4Error):
        fq.fp4q_buffer_sizes(C(), 16, 40)


def test_mm_rules():
    """fp4_mm (MXFP4 operands, K % 64 == 0) and the GEMM-ready scale layout."""
    C = fq.make_cfg
    L = fq.lib()
    mx = C(format="mxfp4")

    def mm(cfg, M=64, N=64, K=128, layout=0, a=FAKE, asc=FAKE, b=FAKE, bsc=FAKE, c=FAKE, ldc=None):
        return _validated(L.fp4_mm(ct.byref(cfg), a, asc, b, bsc, M, N, K, layout, c, N if ldc is None else ldc, None))
    assert mm(C()) == fq.ERR_MODE                                       # NVFP4 operands: not this consumer
    assert mm(mx, layout=2) == fq.ERR_MODE
    assert mm(mx, K=96) == fq.ERR_SHAPE                                 # K % 64
    assert mm(mx, M=-1) == fq.ERR_SHAPE
    assert mm(mx, ldc=32) == fq.ERR_SHAPE                               # ldc < N
    assert mm(mx, K=(1 << 22) + 64) == fq.ERR_UNSUPPORTED
    assert mm(mx, a=None) == fq.ERR_NULL
    assert mm(mx, c=None) == fq.ERR_NULL
    assert mm(mx, a=FAKE_MIS) == fq.ERR_ALIGN
    assert mm(mx, layout=1, asc=FAKE + 4) == fq.ERR_ALIGN
    assert mm(C(format="mxfp4", output_dtype="fp32"), c=FAKE + 2) == fq.ERR_ALIGN
    assert mm(C(format="mxfp4", output_dtype="fp16")) == fq.ERR_DTYPE
    assert mm(mx, M=0, a=None, asc=None, b=None, bsc=None, c=None) == fq.OK
    # the GEMM-ready scale layout: 2 KiB per 256-row tile and 256-value K-tile
    assert fq.fp4q_mx_scales_tiled_bytes(300, 2880) == 2 * 12 * 2048
    assert fq.fp4q_mx_scales_tiled_bytes(0, 64) == 0
    assert _validated(L.fp4_mx_scales_tiled(FAKE, 64, 48, FAKE, None)) == fq.ERR_SHAPE
    assert _validated(L.fp4_mx_scales_tiled(FAKE, 64, 64, FAKE + 4, None)) == fq.ERR_ALIGN
    assert _validated(L.fp4_mx_scales_tiled(None, 64, 64, FAKE, None)) == fq.ERR_NULL
    assert _validated(L.fp4_mx_scales_tiled(None, 0, 64, None, None)) == fq.OK
