"""GPU parity of binary32 sources, binary32 targets and misaligned views
against the CPU oracle, bit for bit, through the C ABI ("fp4-train" README,
Requirements and limits: float32 or bfloat16 input; "MXFP4 weight QAT
recipes", Correctness: fake-quant on bf16 and fp32, dequantise to bf16 and
fp32 targets, fp32 raw-bit fuzz, misaligned views).

A misaligned view is a source whose start and row pitch are multiples of the
element size only (a slice at an odd column of a tensor with an odd row
pitch); the oracle runs on a contiguous copy of the same values.
"""
import zlib

import numpy as np
import pytest
import torch

import block_scaled_fp4_amax_amd as fq
from block_scaled_fp4_amax_amd import workloads as W
from oracle import ref

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fq.lib()


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(a).cuda()


def host(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    a = t.detach().cpu().contiguous().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def canary(shape, dtype=torch.uint8):
    t = torch.empty(shape, dtype=dtype, device="cuda")
    t.view(torch.uint8).fill_(0xA5)
    return t


def same(gpu, want, what):
    gpu, want = np.asarray(gpu), np.asarray(want)
    if gpu.dtype == np.float32 or want.dtype == np.float32:
        gpu = gpu.astype(np.float32).view(np.uint32)
        want = want.astype(np.float32).view(np.uint32)
    gpu = gpu.reshape(want.shape)
    bad = np.flatnonzero(gpu.ravel() != want.ravel())
    assert bad.size == 0, "%s: %d of %d differ; first at flat %d: gpu %s oracle %s" % (
        what, bad.size, want.size, bad[0], hex(int(gpu.ravel()[bad[0]])), hex(int(want.ravel()[bad[0]])))


FMT = {"nvfp4": ("nvfp4", None, "e4m3"), "nvfp4-ue5m3": ("nvfp4", "ue5m3", "ue5m3"), "amdfp4": ("amdfp4", None, "ue5m3")}


def cfgs(fmt, two_level="none", obs=0, sr=False, seed=0, step=0, index_base=0):
    f, sf, osf = FMT[fmt]
    gtl = {"none": "none", "tensorwise": "tensorwise", "outer": "outer_block"}[two_level]
    g = fq.make_cfg(format=f, scale_format=sf, two_level=gtl, outer_block_size=obs,
                    rounding="stochastic" if sr else "rne", seed=seed, step=step, index_base=index_base)
    o = dict(scale_fmt=osf, two_level=two_level, obs=obs, stochastic=sr, seed=seed, step=step, index_base=index_base)
    return g, o


def ydt(name):
    return torch.float32 if name == "fp32" else torch.bfloat16


def check_rowwise(x_dev, x_host, g, o, want_y, ef_seed=None, what=""):
    """qdq (y in want_y) with codes, and quantize into canaries, against the oracle."""
    R, C = x_host.shape
    z0 = None
    if ef_seed is not None:
        z0 = (np.random.default_rng(ef_seed).standard_normal((R, C)) * 0.05).astype(np.float32)
    zo = None if z0 is None else z0.copy()
    want = ref.nv_quantize(x_host, residual=zo, y_dtype=want_y, **o)
    zd = None if z0 is None else torch.from_numpy(z0.copy()).cuda()
    out = fq.fp4_qdq(x_dev, g, residual=zd, with_codes=True, y_dtype=ydt(want_y))
    same(host(out["y"]), want["row_y"], what + " y")
    same(host(out["codes"]), want["row_codes"], what + " codes")
    same(host(out["scales"]), want["row_scales"], what + " scales")
    if "row_outer" in want:
        same(host(out["outer"]), want["row_outer"], what + " outer")
    if z0 is not None:
        same(host(zd), zo, what + " residual")
    zd2 = None if z0 is None else torch.from_numpy(z0.copy()).cuda()
    q = fq.fp4_quantize(x_dev, g, residual=zd2, out={"codes": canary((R, C // 2)), "scales": canary((R, C // 16))})
    same(host(q["codes"]), want["row_codes"], what + " quantize codes")
    same(host(q["scales"]), want["row_scales"], what + " quantize scales")
    if z0 is not None:
        same(host(zd2), zo, what + " quantize residual")


ROW_CASES = [
    # fmt, two_level, obs, sr, ef, shape, index_base
    ("nvfp4", "none", 0, False, False, (50, 192), 0),
    ("nvfp4", "none", 0, True, True, (50, 192), 77),
    ("nvfp4", "tensorwise", 0, False, False, (50, 192), 0),
    ("amdfp4", "tensorwise", 0, True, True, (33, 320), 8),
    ("nvfp4", "outer", 16, False, False, (50, 192), 0),
    ("nvfp4", "outer", 32, True, False, (50, 192), 5),
    ("amdfp4", "outer", 64, True, True, (70, 2880), 3),
    ("nvfp4-ue5m3", "outer", 128, False, False, (50, 256), 0),
]


@pytest.mark.parametrize("y_dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("case", ROW_CASES, ids=lambda c: "-".join(str(v) for v in c[:5]) + "-%dx%d" % c[5])
def test_nv_fp32_source(case, y_dtype):
    fmt, tl, obs, sr, ef, shape, ib = case
    seed = zlib.crc32(repr(case).encode())
    x = W.fp32_weights(seed % 1000, *shape)
    g, o = cfgs(fmt, tl, obs, sr, seed=11, step=2, index_base=ib)
    check_rowwise(dev(x), x, g, o, y_dtype, ef_seed=seed if ef else None, what="%s fp32 source" % fmt)


def test_nv_fp32_edge_values():
    # signed zeros, subnormals, the largest binary32 (beyond bf16's), +-inf and
    # NaN (sanitised), 1 and its binary32 neighbours, values near 6
    vals = np.array([0x00000000, 0x80000000, 0x00000001, 0x807FFFFF, 0x00400000, 0x7F7FFFFF, 0xFF7FFFFF,
                     0x7F800000, 0xFF800000, 0x7FC00001, 0x7F7F0000, 0x7F7F8000, 0x3F800000, 0x3F800001,
                     0x3F7FFFFF, 0x40C00001], np.uint32)
    rng = np.random.default_rng(5)
    for tl, obs in [("none", 0), ("tensorwise", 0), ("outer", 16), ("outer", 32)]:
        for fmt in ("nvfp4", "amdfp4"):
            for sr in (False, True):
                xb = rng.choice(vals, size=(32, 64)).astype(np.uint32)
                xb[:, 16:32] = rng.choice(vals[:5], size=(32, 16))
                x = xb.view(np.float32)
                g, o = cfgs(fmt, tl, obs, sr, seed=3, step=1)
                for y_dtype in ("bf16", "fp32"):
                    check_rowwise(dev(x), x, g, o, y_dtype, what="edge %s %s sr=%d %s" % (fmt, tl, sr, y_dtype))


@pytest.mark.parametrize("y_dtype", ["bf16", "fp32"])
def test_mx_fp32_raw_bit_fuzz(y_dtype):
    xb = W.fp32_raw_bit_blocks(41, 96, 1024)
    x = xb.view(np.float32)
    c, s, y = ref.mx_qdq(x, y_dtype=y_dtype)
    cfg = fq.make_cfg(format="mxfp4")
    out = fq.fp4_qdq(dev(x), cfg, with_codes=True, y_dtype=ydt(y_dtype))
    same(host(out["y"]), y, "MXFP4 fp32 y")
    same(host(out["codes"]), c, "MXFP4 fp32 codes")
    same(host(out["scales"]), s, "MXFP4 fp32 scales")
    q = fq.fp4_quantize(dev(x), cfg, out={"codes": canary((96, 512)), "scales": canary((96, 32))})
    same(host(q["codes"]), c, "MXFP4 fp32 quantize codes")
    same(host(q["scales"]), s, "MXFP4 fp32 quantize scales")


def _fp32_edge_weight():
    """The 8192 x 8192 MXFP4 edge weight widened to binary32, with every finite
    nonzero value given random low significand bits (inf / NaN / zeros kept)."""
    xb = W.mx_weight_8192_edges()
    x = W.from_bf16(xb).copy()
    bits = x.view(np.uint32)
    low = np.random.default_rng(8).integers(0, 1 << 16, bits.shape, dtype=np.uint32)
    finite_nz = ((bits & np.uint32(0x7F800000)) != np.uint32(0x7F800000)) & ((bits & np.uint32(0x7FFFFFFF)) != 0)
    bits[finite_nz] |= low[finite_nz]
    return x


def test_mx_fp32_fake_quant_8192_full_size():
    x = _fp32_edge_weight()
    c, s, y = ref.mx_qdq(x, y_dtype="fp32")
    cfg = fq.make_cfg(format="mxfp4")
    xd = dev(x)
    out = fq.fp4_qdq(xd, cfg, with_codes=True)
    assert out["y"].dtype == torch.float32
    same(host(out["y"]), y, "MXFP4 fp32 8192 y")
    same(host(out["codes"]), c, "MXFP4 fp32 8192 codes")
    same(host(out["scales"]), s, "MXFP4 fp32 8192 scales")
    yd = fq.fp4_dequantize(out["codes"], out["scales"], None, 8192, 8192, cfg, dtype=torch.float32)
    same(host(yd), y, "MXFP4 fp32 8192 dequantize")


def test_dequantize_fp32_targets():
    rng = np.random.default_rng(10)
    x = W.to_bf16(rng.standard_normal((128, 192)).astype(np.float32) * np.float32(0.02))
    for fmt in ("nvfp4", "amdfp4"):
        for tl, obs, o2d, ck in (("none", 0, False, "none"), ("tensorwise", 0, False, "tensorwise"),
                                 ("outer", 64, False, "1d"), ("outer", 64, True, "2d_t")):
            f, sf, osf = FMT[fmt]
            g = fq.make_cfg(format=f, scale_format=sf, two_level={"none": "none", "tensorwise": "tensorwise",
                                                                  "outer": "outer_block"}[tl],
                            outer_block_size=obs, outer_2d=o2d)
            want = ref.nv_quantize(x, cols=True, scale_fmt=osf, two_level=tl, obs=obs, outer_2d=o2d, y_dtype="fp32")
            ro = want.get("row_outer")
            co = want.get("col_outer", ro)
            t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
            y = fq.fp4_dequantize(t(want["row_codes"]), t(want["row_scales"]), t(ro), 128, 192, g, dtype=torch.float32)
            same(host(y), want["row_y"], "%s %s fp32 row dequant" % (fmt, tl))
            yc = fq.fp4_dequantize(t(want["col_codes"]), t(want["col_scales"]), t(co), 192, 128, g,
                                   outer_transposed=(ck == "2d_t"), dtype=torch.float32)
            same(host(yc), want["col_y"], "%s %s fp32 col dequant" % (fmt, tl))
    c, s, y = ref.mx_qdq(W.mx_weight_8192_edges(rows=64, cols=512), y_dtype="fp32")
    yd = fq.fp4_dequantize(torch.from_numpy(c).cuda(), torch.from_numpy(s).cuda(), None, 64, 512,
                           fq.make_cfg(format="mxfp4"), dtype=torch.float32)
    same(host(yd), y, "MXFP4 fp32 dequant")


# ---------------------------------------------------------------- misaligned views
def _view(full_host, off, C):
    """(device view of full[:, off:off + C], contiguous host copy)."""
    return dev(full_host)[:, off:off + C], np.ascontiguousarray(full_host[:, off:off + C])


VIEW_MODES = [
    # fmt, two_level, obs, sr, ef
    ("nvfp4", "none", 0, False, False),
    ("nvfp4", "tensorwise", 0, True, True),
    ("nvfp4", "outer", 32, True, False),
    ("amdfp4", "outer", 64, False, True),
]


@pytest.mark.parametrize("mode", VIEW_MODES, ids=lambda m: "-".join(str(v) for v in m))
@pytest.mark.parametrize("off,pad", [(1, 3), (3, 8), (7, 1), (8, 5)])
def test_bf16_misaligned_views(mode, off, pad):
    fmt, tl, obs, sr, ef = mode
    R, C = 45, 320
    rng = np.random.default_rng(off * 100 + pad)
    full = W.to_bf16((rng.standard_normal((R, C + off + pad)) * 0.05).astype(np.float32))
    full[:, off + 5] = W.to_bf16(np.full(R, 300.0, np.float32))
    xv, xh = _view(full, off, C)
    assert (xv.data_ptr() % 16 != 0) or (xv.stride(0) * 2) % 16 != 0
    g, o = cfgs(fmt, tl, obs, sr, seed=4, step=9, index_base=3)
    check_rowwise(xv, xh, g, o, "bf16", ef_seed=off if ef else None, what="bf16 view off=%d pad=%d" % (off, pad))


@pytest.mark.parametrize("off,pad", [(1, 3), (2, 1), (3, 6), (4, 3)])
def test_fp32_misaligned_views(off, pad):
    R, C = 40, 256
    full = W.fp32_weights(off * 10 + pad, R, C + off + pad)
    xv, xh = _view(full, off, C)
    for mode in VIEW_MODES:
        fmt, tl, obs, sr, ef = mode
        g, o = cfgs(fmt, tl, obs, sr, seed=6, step=1)
        check_rowwise(xv, xh, g, o, "fp32", ef_seed=7 if ef else None, what="fp32 view %s off=%d" % (mode, off))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("off,pad", [(1, 1), (5, 3), (8, 7)])
def test_mx_misaligned_views(dtype, off, pad):
    R, C = 32, 512
    if dtype == "bf16":
        full = W.mx_weight_8192_edges(rows=R, cols=1024)[:, :C + off + pad]
    else:
        full = W.fp32_raw_bit_blocks(off + 20 * pad, R, C + 32).view(np.float32)[:, :C + off + pad]
    full = np.ascontiguousarray(full)
    xv, xh = _view(full, off, C)
    c, s, y = ref.mx_qdq(xh, y_dtype=dtype)
    cfg = fq.make_cfg(format="mxfp4")
    out = fq.fp4_qdq(xv, cfg, with_codes=True)
    same(host(out["y"]), y, "MX %s view y" % dtype)
    same(host(out["codes"]), c, "MX %s view codes" % dtype)
    same(host(out["scales"]), s, "MX %s view scales" % dtype)
