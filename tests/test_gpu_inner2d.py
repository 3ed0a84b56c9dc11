"""GPU parity of 16 x 16 inner scaling ("Block-Scaled FP8 and FP4 Weight
Quantization", section 6: a square tile shares one scale, and the columnwise
codes and scales follow from the rowwise ones by transposition) against the CPU
oracle, bit for bit, through the C ABI: packed codes, replicated scale bytes,
outer FP32 scales, dequantised bf16 and residuals.  Inputs are seeded and
synthetic; output buffers are pre-filled with 0xA5 where the binding allows.
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
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def host(t, dtype):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.detach().cpu().contiguous().numpy().view(dtype)


def canary(shape):
    t = torch.empty(shape, dtype=torch.uint8, device="cuda")
    t.fill_(0xA5)
    return t


def same(gpu, want, what):
    gpu = np.asarray(gpu)
    want = np.asarray(want)
    if gpu.dtype == np.float32:
        gpu = gpu.view(np.uint32)
        want = want.astype(np.float32).view(np.uint32)
    gpu = gpu.reshape(want.shape)
    bad = np.flatnonzero(gpu.ravel() != want.ravel())
    assert bad.size == 0, "%s: %d of %d differ; first at flat %d: gpu %s oracle %s" % (
        what, bad.size, want.size, bad[0], hex(int(gpu.ravel()[bad[0]])), hex(int(want.ravel()[bad[0]])))


FMT = {"nvfp4": ("nvfp4", None, "e4m3"), "nvfp4-ue5m3": ("nvfp4", "ue5m3", "ue5m3"), "amdfp4": ("amdfp4", None, "ue5m3")}
OUTER = {"none": ("none", 0, False), "tensorwise": ("tensorwise", 0, False), "2d": ("outer_block", 64, True)}
ORC_OUTER = {"none": ("none", 0, False), "tensorwise": ("tensorwise", 0, False), "2d": ("outer", 64, True)}


def cfgs(fmt, outer, sr=False, seed=0, step=0, index_base=0):
    f, sf, osf = FMT[fmt]
    tl, obs, o2d = OUTER[outer]
    g = fq.make_cfg(format=f, scale_format=sf, two_level=tl, outer_block_size=obs, outer_2d=o2d,
                    rounding="stochastic" if sr else "rne", seed=seed, step=step, index_base=index_base,
                    inner_2d=True)
    otl, oobs, oo2d = ORC_OUTER[outer]
    o = dict(scale_fmt=osf, two_level=otl, obs=oobs, outer_2d=oo2d, stochastic=sr, seed=seed, step=step,
             index_base=index_base, inner_2d=True)
    return g, o


def weight(rng, shape, outlier_cols=1, outlier_rows=1):
    """N(0, 0.02) rows with a per-row magnitude spread, plus outlier columns
    and rows (x1000 / x200) so tiles with and without an outlier coexist."""
    a = rng.standard_normal(shape).astype(np.float32) * np.float32(0.02)
    a *= np.exp(rng.standard_normal((shape[0], 1))).astype(np.float32)
    for c in rng.choice(shape[1], size=outlier_cols, replace=False):
        a[:, c] *= np.float32(1000)
    for r in rng.choice(shape[0], size=outlier_rows, replace=False):
        a[r, :] *= np.float32(200)
    return W.to_bf16(a)


def nibble_transpose(codes, R, C):
    """[R, C/2] packed codes -> the packed codes of the transpose, [C, R/2]."""
    c = np.asarray(codes, np.uint8).reshape(R, C // 2)
    n = np.empty((R, C), np.uint8)
    n[:, 0::2] = c & 0x0F
    n[:, 1::2] = c >> 4
    t = np.ascontiguousarray(n.T)
    return (t[:, 0::2] | (t[:, 1::2] << 4)).astype(np.uint8)


CT_CASES = [
    # fmt, outer, sr, ef, shape
    ("nvfp4", "2d", False, False, (128, 192)),
    ("nvfp4", "2d", True, True, (192, 128)),
    ("amdfp4", "2d", True, False, (128, 320)),
    ("nvfp4-ue5m3", "2d", False, True, (64, 64)),
    ("nvfp4", "none", False, False, (80, 48)),
    ("nvfp4", "none", True, True, (144, 208)),
    ("amdfp4", "none", False, False, (16, 16)),
    ("nvfp4", "tensorwise", False, False, (112, 96)),
    ("nvfp4-ue5m3", "tensorwise", True, True, (48, 400)),
]


@pytest.mark.parametrize("case", CT_CASES, ids=lambda c: "-".join(str(v) for v in c[:4]) + "-%dx%d" % c[4])
def test_cast_transpose_inner_2d(case):
    fmt, outer, sr, ef, shape = case
    R, C = shape
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    x = weight(rng, shape)
    z0 = (rng.standard_normal(shape) * 0.003).astype(np.float32) if ef else None
    g, o = cfgs(fmt, outer, sr, seed=7, step=3)
    zo = None if z0 is None else z0.copy()
    want = ref.nv_quantize(x, residual=zo, cols=True, want_y=False, **o)
    zd = None if z0 is None else torch.from_numpy(z0.copy()).cuda()
    out = fq.fp4_cast_transpose(dev(x), g, residual=zd, out={
        "row_codes": canary((R, C // 2)), "row_scales": canary((R, C // 16)),
        "col_codes": canary((C, R // 2)), "col_scales": canary((C, R // 16))})
    got = {k: host(out[k], np.uint8) for k in ("row_codes", "row_scales", "col_codes", "col_scales")}
    for k, v in got.items():
        same(v, want[k], k)
    if "row_outer" in want:
        same(host(out["row_outer"], np.float32), want["row_outer"], "row_outer")
    if ef:
        same(host(zd, np.float32), zo, "residual")
    # the columnwise buffers are the transposes of the rowwise ones
    same(got["col_codes"], nibble_transpose(got["row_codes"], R, C), "col codes = transpose of row codes")
    same(got["col_scales"], np.ascontiguousarray(got["row_scales"].reshape(R, C // 16)[::16].T.repeat(16, axis=0)),
         "col scales = transpose of row scales")


ROW_CASES = [
    # fmt, outer, sr, ef, shape
    ("nvfp4", "none", False, False, (48, 96)),
    ("nvfp4", "tensorwise", True, True, (96, 160)),
    ("amdfp4", "2d", False, True, (128, 192)),
    ("nvfp4", "2d", True, False, (192, 64)),
]


@pytest.mark.parametrize("case", ROW_CASES, ids=lambda c: "-".join(str(v) for v in c[:4]) + "-%dx%d" % c[4])
def test_rowwise_quantize_and_qdq_inner_2d(case):
    fmt, outer, sr, ef, shape = case
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    x = weight(rng, shape)
    z0 = (rng.standard_normal(shape) * 0.003).astype(np.float32) if ef else None
    g, o = cfgs(fmt, outer, sr, seed=2, step=9)
    zo = None if z0 is None else z0.copy()
    want = ref.nv_quantize(x, residual=zo, **o)
    # quantise
    zd = None if z0 is None else torch.from_numpy(z0.copy()).cuda()
    q = fq.fp4_quantize(dev(x), g, residual=zd)
    same(host(q["codes"], np.uint8), want["row_codes"], "quantize codes")
    same(host(q["scales"], np.uint8), want["row_scales"], "quantize scales")
    if "row_outer" in want:
        same(host(q["outer"], np.float32), want["row_outer"], "quantize outer")
    if ef:
        same(host(zd, np.float32), zo, "quantize residual")
    # quantise-dequantise
    zd = None if z0 is None else torch.from_numpy(z0.copy()).cuda()
    d = fq.fp4_qdq(dev(x), g, residual=zd, with_codes=True)
    same(host(d["y"], np.uint16), want["row_y"], "qdq y")
    same(host(d["codes"], np.uint8), want["row_codes"], "qdq codes")
    if ef:
        same(host(zd, np.float32), zo, "qdq residual")
    # the stored buffers dequantise to the same bf16 in both directions
    wc = ref.nv_quantize(x, residual=None if z0 is None else z0.copy(), cols=True, **o)
    ro = wc.get("row_outer")
    y = fq.fp4_dequantize(torch.from_numpy(wc["row_codes"]).cuda(), torch.from_numpy(wc["row_scales"]).cuda(),
                          None if ro is None else torch.from_numpy(np.ascontiguousarray(ro)).cuda(),
                          shape[0], shape[1], g)
    same(host(y, np.uint16), wc["row_y"], "dequantize rows")
    yc = fq.fp4_dequantize(torch.from_numpy(wc["col_codes"]).cuda(), torch.from_numpy(wc["col_scales"]).cuda(),
                           None if ro is None else torch.from_numpy(np.ascontiguousarray(ro)).cuda(),
                           shape[1], shape[0], g, outer_transposed=(outer == "2d"))
    same(host(yc, np.uint16), wc["col_y"], "dequantize cols")
    same(host(yc, np.uint16), np.ascontiguousarray(wc["row_y"].T), "columnwise effective weight = transpose")


def test_inner_2d_edge_values():
    vals = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x0040, 0x7F7F, 0xFF7F, 0x7F80, 0xFF80, 0x7FC0, 0x3F80, 0xBF80,
                     0x4013, 0x2000, 0x1000, 0x0100], np.uint16)
    rng = np.random.default_rng(13)
    x = rng.choice(vals, size=(128, 128)).astype(np.uint16)
    x[:64, 64:] = rng.choice(vals[:6], size=(64, 64))      # zeros, subnormals and the largest finite values
    x[64:, :64] = 0                                         # an all-zero 64 x 64 tile
    x[16:32, 0:16] = 0x0001                                 # a 16 x 16 tile of the smallest subnormal
    for fmt in ("nvfp4", "amdfp4"):
        for outer in ("none", "tensorwise", "2d"):
            for sr in (False, True):
                g, o = cfgs(fmt, outer, sr=sr, seed=11, step=2)
                want = ref.nv_quantize(x, cols=True, want_y=False, **o)
                out = fq.fp4_cast_transpose(dev(x), g)
                for k in ("row_codes", "row_scales", "col_codes", "col_scales", "row_outer"):
                    if k in want:
                        same(host(out[k], np.float32 if "outer" in k else np.uint8), want[k],
                             "%s %s sr=%s %s" % (fmt, outer, sr, k))


def test_grouped_inner_2d_sr_ef_uneven_groups():
    rng = np.random.default_rng(14)
    rows = [64, 128, 0, 192]
    C = 192
    x = weight(rng, (sum(rows), C), outlier_cols=2, outlier_rows=3)
    z0 = (rng.standard_normal(x.shape) * 0.003).astype(np.float32)
    g = fq.make_cfg(format="nvfp4", two_level="outer_block", outer_block_size=64, outer_2d=True,
                    rounding="stochastic", seed=5, step=2, inner_2d=True)
    zo = z0.copy()
    want = ref.nv_quantize_grouped(x, rows, two_level="outer", obs=64, outer_2d=True, stochastic=True, seed=5, step=2,
                                   residual=zo, inner_2d=True)
    zd = torch.from_numpy(z0.copy()).cuda()
    out = fq.fp4_cast_transpose_grouped(dev(x), rows, g, residual=zd)
    for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
        same(host(out[k], np.uint8), want[k], "grouped " + k)
    same(host(out["row_outer"], np.float32), want["row_outer"], "grouped outer")
    same(host(zd, np.float32), zo, "grouped residual")


def test_weight_4096_inner_2d_outer_2d_full_size():
    """The 4096 x 4096 weight (N(0, 0.02), 0.5% of columns x1000) under the
    transpose-consistent weight recipe: 16 x 16 E4M3 inner tiles inside 64 x 64
    FP32 outer tiles, RTNE, both directions; every output byte compared."""
    x = W.weight_4096_outlier_cols()
    g, o = cfgs("nvfp4", "2d")
    want = ref.nv_quantize(x, cols=True, want_y=False, **o)
    out = fq.fp4_cast_transpose(dev(x), g)
    for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
        same(host(out[k], np.uint8), want[k], "4096 inner-2D " + k)
    same(host(out["row_outer"], np.float32), want["row_outer"], "4096 inner-2D outer")
