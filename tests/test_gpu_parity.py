"""GPU parity: every HIP entry point against the CPU oracle, bit for bit.

The bar is 0 ULP / byte equality on packed codes, scale bytes, outer FP32
scales, dequantised bf16 and residuals.  Inputs are seeded and synthetic
(block_scaled_fp4_amax_amd.workloads); the oracle sees exactly the same
arrays.  Output buffers are pre-filled with 0xA5 where the binding allows, so
unwritten bytes show up as mismatches.
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


def canary(shape, dtype=torch.uint8):
    t = torch.empty(shape, dtype=dtype, device="cuda")
    t.view(torch.uint8).fill_(0xA5)
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


def cfgs(fmt, two_level="none", obs=0, outer_2d=False, sr=False, seed=0, step=0, index_base=0, outer_mode=0):
    f, sf, osf = FMT[fmt]
    gtl = {"none": "none", "tensorwise": "tensorwise", "outer": "outer_block"}[two_level]
    g = fq.make_cfg(format=f, scale_format=sf, two_level=gtl, outer_block_size=obs, outer_2d=outer_2d,
                    rounding="stochastic" if sr else "rne", seed=seed, step=step, index_base=index_base,
                    outer_mode=outer_mode)
    o = dict(scale_fmt=osf, two_level=two_level, obs=obs, outer_2d=outer_2d, stochastic=sr, seed=seed, step=step,
             index_base=index_base)
    return g, o


def rand_bf16(rng, shape, scale=1.0, rowscale=True):
    a = rng.standard_normal(shape).astype(np.float32) * np.float32(scale)
    if rowscale:
        a *= np.exp(rng.standard_normal((shape[0], 1))).astype(np.float32)
    return W.to_bf16(a)


# =============================================================== MXFP4
def test_mx_all_65536_bf16_patterns():
    v = np.arange(65536, dtype=np.uint16)
    blocks = []
    x = np.zeros((65536, 32), np.uint16)
    x[:, 5] = v
    blocks.append(x)
    for k0 in (-126, 0, 125):
        a = np.zeros((65536, 32), np.uint16)
        a[:, 0] = W.to_bf16(np.float32([6.0 * 2.0 ** k0]))[0]
        a[:, 17] = v
        blocks.append(a)
    x = np.concatenate(blocks)
    c, s, y = ref.mx_qdq(x)
    out = fq.fp4_qdq(dev(x), fq.make_cfg(format="mxfp4"), with_codes=True)
    same(host(out["y"], np.uint16), y, "y")
    same(host(out["codes"], np.uint8), c, "codes")
    same(host(out["scales"], np.uint8), s, "scales")


@pytest.mark.parametrize("shape,ld", [((1, 32), 32), ((37, 96), 104), ((513, 256), 256), ((3, 4096), 4160)])
def test_mx_shapes_and_strides(shape, ld):
    rng = np.random.default_rng(sum(shape))
    R, C = shape
    full = rand_bf16(rng, (R, ld), 0.02)
    full[:, ::7] = rng.choice(W.TINY_BF16, full[:, ::7].shape)
    x = np.ascontiguousarray(full[:, :C])
    c, s, y = ref.mx_qdq(x)
    xd = dev(full)[:, :C]
    out = fq.fp4_qdq(xd, fq.make_cfg(format="mxfp4"), with_codes=True)
    same(host(out["y"], np.uint16), y, "y")
    same(host(out["codes"], np.uint8), c, "codes")
    same(host(out["scales"], np.uint8), s, "scales")
    q = fq.fp4_quantize(xd, fq.make_cfg(format="mxfp4"), out={"codes": canary((R, C // 2)), "scales": canary((R, C // 32))})
    same(host(q["codes"], np.uint8), c, "quantize codes")
    same(host(q["scales"], np.uint8), s, "quantize scales")


def test_mx_fake_quant_8192_full_size():
    x = W.mx_weight_8192_edges()
    c, s, y = ref.mx_qdq(x)
    xd = dev(x)
    out = fq.fp4_qdq(xd, fq.make_cfg(format="mxfp4"))
    same(host(out["y"], np.uint16), y, "MXFP4 y")
    out2 = fq.fp4_qdq(xd, fq.make_cfg(format="mxfp4"), with_codes=True)
    same(host(out2["y"], np.uint16), y, "MXFP4 y (with codes)")
    same(host(out2["codes"], np.uint8), c, "MXFP4 codes")
    same(host(out2["scales"], np.uint8), s, "MXFP4 scales")
    yd = fq.fp4_dequantize(out2["codes"], out2["scales"], None, 8192, 8192, fq.make_cfg(format="mxfp4"))
    same(host(yd, np.uint16), y, "MXFP4 dequantize")


# =============================================================== NVFP4 / AMD-FP4 rowwise
ROW_CASES = [
    # fmt, two_level, obs, sr, ef, shape, index_base
    ("nvfp4", "none", 0, False, False, (50, 192), 0),
    ("nvfp4", "none", 0, True, True, (50, 192), 77),
    ("nvfp4", "tensorwise", 0, False, False, (50, 192), 0),
    ("nvfp4", "tensorwise", 0, True, True, (33, 320), 8),
    ("amdfp4", "tensorwise", 0, False, False, (256, 256), 0),
    ("nvfp4", "outer", 16, False, False, (50, 192), 0),
    ("nvfp4", "outer", 32, True, False, (50, 192), 5),
    ("nvfp4", "outer", 64, False, True, (50, 192), 0),
    ("amdfp4", "outer", 64, True, True, (70, 2880), 3),
    ("nvfp4-ue5m3", "outer", 64, False, False, (70, 2880), 0),
    ("nvfp4", "outer", 128, False, False, (50, 256), 0),
    ("amdfp4", "outer", 128, True, False, (50, 256), 0),
    ("nvfp4", "tensorwise", 0, True, True, (600, 512), 3),      # above the one-launch size: amax passes
    ("amdfp4", "tensorwise", 0, False, False, (512, 512), 0),   # exactly the one-launch limit
    # small tensors with a residual across many workgroups: the residual is
    # rewritten in place, so these must take the amax passes, not the one-launch form
    ("nvfp4", "tensorwise", 0, True, True, (512, 512), 1),
    ("amdfp4", "tensorwise", 0, False, True, (384, 640), 0),
]


@pytest.mark.parametrize("case", ROW_CASES, ids=lambda c: "-".join(str(v) for v in c[:5]) + "-%dx%d" % c[5])
def test_rowwise_quantize_and_qdq(case):
    fmt, tl, obs, sr, ef, shape, ib = case
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    x = rand_bf16(rng, shape)
    x[rng.integers(0, shape[0]), :] = W.to_bf16(W.from_bf16(x[0]) * np.float32(1e4))
    z0 = (rng.standard_normal(shape) * 0.05).astype(np.float32) if ef else None
    g, o = cfgs(fmt, tl, obs, False, sr, seed=11, step=2, index_base=ib)
    zo = None if z0 is None else z0.copy()
    want = ref.nv_quantize(x, residual=zo, **o)
    # qdq (y + codes + scales + outer + residual)
    zd = None if z0 is None else torch.from_numpy(z0.copy()).cuda()
    out = fq.fp4_qdq(dev(x), g, residual=zd, with_codes=True)
    same(host(out["y"], np.uint16), want["row_y"], "y")
    same(host(out["codes"], np.uint8), want["row_codes"], "codes")
    same(host(out["scales"], np.uint8), want["row_scales"], "scales")
    if "row_outer" in want:
        same(host(out["outer"], np.float32), want["row_outer"], "outer")
    if ef:
        same(host(zd, np.float32), zo, "residual")
    # quantize only, canary-filled outputs
    zd2 = None if z0 is None else torch.from_numpy(z0.copy()).cuda()
    R, C = shape
    q = fq.fp4_quantize(dev(x), g, residual=zd2, out={"codes": canary((R, C // 2)), "scales": canary((R, C // 16))})
    same(host(q["codes"], np.uint8), want["row_codes"], "quantize codes")
    same(host(q["scales"], np.uint8), want["row_scales"], "quantize scales")
    if ef:
        same(host(zd2, np.float32), zo, "quantize residual")


def _every_bf16_at_every_scale(scale_fmt):
    """Blocks of 16: element 0 is 6 * d_c for inner scale code c (so the block's scale is c), elements 1..15
    run through every finite bf16 value of magnitude <= 6 * d_c, both signs; every code c that such an
    amax can reach."""
    mags = np.arange(0x0000, 0x7F80, dtype=np.uint32)                      # finite non-negative bf16
    fmag = (mags << 16).view(np.float32)
    blocks = []
    for c in range(1, 255):
        d = np.float32(ref.scale_decode(scale_fmt, c))
        if not np.isfinite(d) or d <= 0:
            continue
        amax = np.float32(6) * d
        ab = W.to_bf16(np.array([amax], np.float32))
        if W.from_bf16(ab)[0] != amax or ref.scale_encode(scale_fmt, float(amax / np.float32(6))) != c:
            continue
        v = mags[fmag <= amax].astype(np.uint16)
        v = np.concatenate([v, v | np.uint16(0x8000)])
        n = -(-v.size // 15) * 15
        v = np.concatenate([v, np.zeros(n - v.size, np.uint16)]).reshape(-1, 15)
        blocks.append(np.concatenate([np.full((v.shape[0], 1), ab[0], np.uint16), v], axis=1))
    x = np.concatenate(blocks).reshape(-1)
    cols = 1024
    x = np.concatenate([x, np.zeros(-x.size % cols, np.uint16)]).reshape(-1, cols)
    return x


@pytest.mark.parametrize("fmt", ["nvfp4", "nvfp4-ue5m3"])
def test_rne_every_bf16_at_every_scale_code(fmt):
    # the RNE inner quantisation (binary32 quotient by the decoded scale, E2M1 round to nearest even) on
    # every finite bf16 value against every inner scale code it can meet
    f, sf, osf = FMT[fmt]
    x = _every_bf16_at_every_scale(osf)
    g, o = cfgs(fmt, "none")
    want = ref.nv_quantize(x, **o)
    R, C = x.shape
    q = fq.fp4_quantize(dev(x), g, out={"codes": canary((R, C // 2)), "scales": canary((R, C // 16))})
    same(host(q["scales"], np.uint8), want["row_scales"], "scales")
    same(host(q["codes"], np.uint8), want["row_codes"], "codes")
    xt = np.ascontiguousarray(x[: R // 64 * 64])                 # the tile kernel, both directions
    out = fq.fp4_cast_transpose(dev(xt), g)
    want2 = ref.nv_quantize(xt, cols=True, want_y=False, **o)
    for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
        same(host(out[k], np.uint8), want2[k], "cast-transpose " + k)


def test_tensorwise_qdq_256_full_size():
    x = W.tensorwise_input_256()
    g, o = cfgs("nvfp4", "tensorwise")
    want = ref.nv_quantize(x, **o)
    out = fq.fp4_qdq(dev(x), g, with_codes=True)
    same(host(out["y"], np.uint16), want["row_y"], "tensorwise y")
    same(host(out["codes"], np.uint8), want["row_codes"], "tensorwise codes")
    same(host(out["scales"], np.uint8), want["row_scales"], "tensorwise scales")
    same(host(out["outer"], np.float32), want["row_outer"], "tensorwise global scale")


def test_rowwise_2d_outer_qdq():
    rng = np.random.default_rng(4)
    x = rand_bf16(rng, (192, 320), 0.02)
    for fmt, sr in (("nvfp4", False), ("amdfp4", True)):
        g, o = cfgs(fmt, "outer", 64, True, sr, seed=3, step=1)
        z0 = (rng.standard_normal(x.shape) * 0.01).astype(np.float32)
        zo = z0.copy()
        want = ref.nv_quantize(x, residual=zo, **o)
        zd = torch.from_numpy(z0.copy()).cuda()
        out = fq.fp4_qdq(dev(x), g, residual=zd, with_codes=True)
        same(host(out["y"], np.uint16), want["row_y"], "y")
        same(host(out["codes"], np.uint8), want["row_codes"], "codes")
        same(host(out["outer"], np.float32), want["row_outer"], "outer")
        same(host(zd, np.float32), zo, "residual")


# =============================================================== cast-transpose
CT_CASES = [
    # fmt, two_level, obs, outer_2d, sr, ef, shape
    ("nvfp4", "outer", 64, True, False, False, (128, 192)),
    ("nvfp4", "outer", 64, True, True, True, (128, 192)),
    ("amdfp4", "outer", 64, True, False, False, (192, 128)),
    ("nvfp4", "outer", 64, False, False, False, (128, 128)),
    ("amdfp4", "outer", 64, False, True, False, (128, 2880)),
    ("amdfp4", "outer", 32, False, True, True, (96, 160)),
    ("nvfp4", "outer", 16, False, False, False, (48, 80)),
    ("nvfp4", "none", 0, False, False, False, (80, 48)),
    ("nvfp4", "none", 0, False, True, True, (144, 208)),
    ("nvfp4", "tensorwise", 0, False, False, False, (80, 48)),
    ("nvfp4-ue5m3", "tensorwise", 0, False, True, True, (112, 96)),
    ("amdfp4", "outer", 128, False, True, False, (256, 384)),
    ("nvfp4", "outer", 128, False, False, True, (128, 256)),
    ("nvfp4", "outer", 128, False, True, True, (384, 128)),
]


@pytest.mark.parametrize("case", CT_CASES, ids=lambda c: "-".join(str(v) for v in c[:6]) + "-%dx%d" % c[6])
def test_cast_transpose(case):
    fmt, tl, obs, o2d, sr, ef, shape = case
    R, C = shape
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    x = rand_bf16(rng, shape, 0.02)
    x[:, rng.integers(0, C)] = W.to_bf16(W.from_bf16(x[:, 0]) * np.float32(1000))
    z0 = (rng.standard_normal(shape) * 0.003).astype(np.float32) if ef else None
    g, o = cfgs(fmt, tl, obs, o2d, sr, seed=7, step=3, index_base=0)
    zo = None if z0 is None else z0.copy()
    want = ref.nv_quantize(x, residual=zo, cols=True, want_y=False, **o)
    zd = None if z0 is None else torch.from_numpy(z0.copy()).cuda()
    out = fq.fp4_cast_transpose(dev(x), g, residual=zd, out={
        "row_codes": canary((R, C // 2)), "row_scales": canary((R, C // 16)),
        "col_codes": canary((C, R // 2)), "col_scales": canary((C, R // 16))})
    for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
        same(host(out[k], np.uint8), want[k], k)
    if "row_outer" in want:
        same(host(out["row_outer"], np.float32), want["row_outer"], "row_outer")
    if "col_outer" in want:
        same(host(out["col_outer"], np.float32), want["col_outer"], "col_outer")
    if ef:
        same(host(zd, np.float32), zo, "residual")


def test_cast_transpose_strided_source():
    rng = np.random.default_rng(9)
    full = rand_bf16(rng, (128, 200), 0.02)
    x = np.ascontiguousarray(full[:, :192])
    g, o = cfgs("nvfp4", "outer", 64, True)
    want = ref.nv_quantize(x, cols=True, want_y=False, **o)
    out = fq.fp4_cast_transpose(dev(full)[:, :192], g)
    for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
        same(host(out[k], np.uint8), want[k], k)


def test_cast_transpose_edge_values():
    vals = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x0040, 0x7F7F, 0xFF7F, 0x7F80, 0xFF80, 0x7FC0, 0x3F80, 0xBF80,
                     0x4013, 0x2000, 0x1000, 0x0100], np.uint16)
    rng = np.random.default_rng(3)
    x = rng.choice(vals, size=(128, 128)).astype(np.uint16)
    x[:64, 64:] = rng.choice(vals[:6], size=(64, 64))      # a tile of zeros / subnormals
    x[64:, :64] = 0                                         # an all-zero tile
    # stochastic rounding too: blocks holding both 0x7F7F and 0x0001 give quotients below the binary32
    # normal range, where only "t > 0" and "u16 == 0" decide the code
    for fmt in ("nvfp4", "amdfp4"):
        for tl, obs, o2d in (("none", 0, False), ("tensorwise", 0, False), ("outer", 64, True), ("outer", 64, False),
                             ("outer", 16, False)):
            for sr in (False, True):
                g, o = cfgs(fmt, tl, obs, o2d, sr=sr, seed=11, step=2)
                want = ref.nv_quantize(x, cols=True, want_y=False, **o)
                out = fq.fp4_cast_transpose(dev(x), g)
                for k in ("row_codes", "row_scales", "col_codes", "col_scales", "row_outer", "col_outer"):
                    if k in want:
                        same(host(out[k], np.float32 if "outer" in k else np.uint8), want[k],
                             "%s %s sr=%s %s" % (fmt, tl, sr, k))


def test_precomputed_outer_equals_recompute():
    rng = np.random.default_rng(5)
    x = rand_bf16(rng, (128, 192), 0.02)
    for o2d in (True, False):
        g, _ = cfgs("nvfp4", "outer", 64, o2d)
        a = fq.fp4_cast_transpose(dev(x), g)
        g1, _ = cfgs("nvfp4", "outer", 64, o2d, outer_mode=1)
        b = fq.fp4_cast_transpose(dev(x), g1, row_outer=a["row_outer"].clone(),
                                  col_outer=None if o2d else a["col_outer"].clone())
        for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
            same(host(b[k], np.uint8), host(a[k], np.uint8), "given outer " + k)


def test_amdfp4_is_nvfp4_with_ue5m3_and_deterministic():
    rng = np.random.default_rng(6)
    x = rand_bf16(rng, (128, 192), 0.02)
    ga, _ = cfgs("amdfp4", "outer", 64, True, True, seed=1, step=1)
    gn, _ = cfgs("nvfp4-ue5m3", "outer", 64, True, True, seed=1, step=1)
    a = fq.fp4_cast_transpose(dev(x), ga)
    b = fq.fp4_cast_transpose(dev(x), gn)
    c = fq.fp4_cast_transpose(dev(x), ga)
    for k in ("row_codes", "row_scales", "col_codes", "col_scales", "row_outer"):
        dt = np.float32 if "outer" in k else np.uint8
        same(host(a[k], dt), host(b[k], dt), "amd vs nv-ue5m3 " + k)
        same(host(a[k], dt), host(c[k], dt), "rerun " + k)


def test_columnwise_is_rowwise_of_transpose_on_gpu():
    rng = np.random.default_rng(8)
    x = rand_bf16(rng, (128, 192), 0.02)
    for o2d in (True, False):
        g, _ = cfgs("nvfp4", "outer", 64, o2d)
        a = fq.fp4_cast_transpose(dev(x), g)
        b = fq.fp4_cast_transpose(dev(np.ascontiguousarray(x.T)), g)
        same(host(a["col_codes"], np.uint8), host(b["row_codes"], np.uint8), "col(X) vs row(X^T) codes")
        same(host(a["col_scales"], np.uint8), host(b["row_scales"], np.uint8), "col(X) vs row(X^T) scales")


# =============================================================== dequantize
def test_dequantize_nv_all_outer_kinds():
    rng = np.random.default_rng(10)
    x = rand_bf16(rng, (128, 192), 0.02)
    for fmt in ("nvfp4", "amdfp4"):
        for tl, obs, o2d, rk, ck in (("none", 0, False, "none", "none"), ("tensorwise", 0, False, "tensorwise", "tensorwise"),
                                     ("outer", 64, False, "1d", "1d"), ("outer", 64, True, "2d", "2d_t")):
            g, o = cfgs(fmt, tl, obs, o2d)
            want = ref.nv_quantize(x, cols=True, **o)
            ro = want.get("row_outer")
            co = want.get("col_outer", ro)
            y = fq.fp4_dequantize(torch.from_numpy(want["row_codes"]).cuda(), torch.from_numpy(want["row_scales"]).cuda(),
                                  None if ro is None else torch.from_numpy(np.ascontiguousarray(ro)).cuda(), 128, 192, g)
            same(host(y, np.uint16), want["row_y"], "%s %s row dequant" % (fmt, tl))
            yc = fq.fp4_dequantize(torch.from_numpy(want["col_codes"]).cuda(), torch.from_numpy(want["col_scales"]).cuda(),
                                   None if co is None else torch.from_numpy(np.ascontiguousarray(co)).cuda(), 192, 128, g,
                                   outer_transposed=(ck == "2d_t"))
            same(host(yc, np.uint16), want["col_y"], "%s %s col dequant" % (fmt, tl))


# =============================================================== full-size workloads
def test_cast_transpose_2d_4096_full_size():
    x = W.weight_4096_outlier_cols()
    g, o = cfgs("nvfp4", "outer", 64, True)
    want = ref.nv_quantize(x, cols=True, want_y=False, **o)
    out = fq.fp4_cast_transpose(dev(x), g)
    for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
        same(host(out[k], np.uint8), want[k], "2D cast-transpose " + k)
    same(host(out["row_outer"], np.float32), want["row_outer"], "2D cast-transpose outer")


def test_cast_transpose_1d_sr_16384x2880_full_size():
    x = W.activations_16384x2880()
    g, o = cfgs("amdfp4", "outer", 64, False, True, seed=7, step=3)
    want = ref.nv_quantize(x, cols=True, want_y=False, **o)
    out = fq.fp4_cast_transpose(dev(x), g)
    for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
        same(host(out[k], np.uint8), want[k], "1D SR cast-transpose " + k)
    same(host(out["row_outer"], np.float32), want["row_outer"], "1D SR cast-transpose row outer")
    same(host(out["col_outer"], np.float32), want["col_outer"], "1D SR cast-transpose col outer")


def test_grouped_sr_ef_32x2880_four_steps():
    """The grouped workload at full size: all 32 experts, every output buffer
    (row / column codes and scale bytes, the per-expert 2D outer scales and the
    in-place residual) at each of the four error-feedback steps, against the
    oracle run on the whole stacked tensor."""
    E, R, C = 32, 2880, 2880
    w = W.experts_32x2880()
    g = fq.make_cfg(format="nvfp4", two_level="outer_block", outer_block_size=64, outer_2d=True, rounding="stochastic",
                    seed=5)
    zd = torch.zeros((E * R, C), dtype=torch.float32, device="cuda")
    z_or = np.zeros((E * R, C), np.float32)
    for t in range(4):
        g.step = t
        out = fq.fp4_cast_transpose_grouped(dev(w), [R] * E, g, residual=zd)
        want = ref.nv_quantize_grouped(w, [R] * E, two_level="outer", obs=64, outer_2d=True, stochastic=True, seed=5,
                                       step=t, residual=z_or)
        for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
            same(host(out[k], np.uint8).reshape(want[k].shape), want[k], "grouped step %d %s" % (t, k))
        same(host(out["row_outer"], np.float32).ravel(), want["row_outer"], "grouped step %d outer" % t)
        same(host(zd, np.float32), z_or, "grouped step %d residual" % t)
        w = W.apply_expert_update(w, W.expert_update(t, w.shape))


def test_grouped_uneven_groups_equal_single_calls():
    rng = np.random.default_rng(12)
    rows = [64, 128, 0, 192]
    C = 128
    x = rand_bf16(rng, (sum(rows), C), 0.02)
    z0 = (rng.standard_normal(x.shape) * 0.01).astype(np.float32)
    for tl, obs, o2d in (("outer", 64, True), ("outer", 64, False), ("none", 0, False)):
        gtl = {"outer": "outer_block", "none": "none"}[tl]
        g = fq.make_cfg(format="nvfp4", two_level=gtl, outer_block_size=obs, outer_2d=o2d, rounding="stochastic",
                        seed=2, step=9)
        zd = torch.from_numpy(z0.copy()).cuda()
        out = fq.fp4_cast_transpose_grouped(dev(x), rows, g, residual=zd)
        rc = host(out["row_codes"], np.uint8)
        cc = host(out["col_codes"], np.uint8)
        rsc = host(out["row_scales"], np.uint8)
        csc = host(out["col_scales"], np.uint8)
        zg = host(zd, np.float32)
        r0 = 0
        co_off = ro_off = 0
        for R in rows:
            zo = z0[r0:r0 + R].copy()
            want = ref.nv_quantize(x[r0:r0 + R], two_level=tl, obs=obs, outer_2d=o2d, stochastic=True, seed=2, step=9,
                                   index_base=r0 * C, residual=zo, cols=True, want_y=False)
            same(rc[r0:r0 + R], want["row_codes"], "%s group rows %d row codes" % (tl, R))
            same(cc[r0 * C // 2:(r0 + R) * C // 2], want["col_codes"].ravel(), "%s group %d col codes" % (tl, R))
            same(rsc[r0:r0 + R], want["row_scales"], "%s group rows %d row scales" % (tl, R))
            same(csc[r0 * C // 16:(r0 + R) * C // 16], want["col_scales"].ravel(), "%s group %d col scales" % (tl, R))
            same(zg[r0:r0 + R], zo, "%s group %d residual" % (tl, R))
            if "row_outer" in want:
                n = want["row_outer"].size
                same(host(out["row_outer"], np.float32)[ro_off:ro_off + n], want["row_outer"].ravel(), "row outer")
                ro_off += n
            if "col_outer" in want:
                n = want["col_outer"].size
                same(host(out["col_outer"], np.float32)[co_off:co_off + n], want["col_outer"].ravel(), "col outer")
                co_off += n
            r0 += R


@pytest.mark.parametrize("tl,obs,o2d", [("outer", 64, True), ("outer", 64, False), ("outer", 16, False),
                                        ("outer", 128, False)])
def test_grouped_more_groups_than_one_launch_holds(tl, obs, o2d):
    """More groups than one launch's group table (64): the call is split into
    several launches, each with its own tile numbering but global row offsets.
    SR + error feedback, groups of uneven height (some empty), every buffer
    against the oracle's grouped quantisation."""
    rng = np.random.default_rng(13 + obs)
    step = 64 if (tl == "outer" and o2d) or obs == 64 else obs
    rows = list(rng.choice([0, step, 2 * step, 3 * step], size=130))
    C = 128
    x = rand_bf16(rng, (sum(rows), C), 0.02)
    z0 = (rng.standard_normal(x.shape) * 0.01).astype(np.float32)
    g = fq.make_cfg(format="nvfp4", two_level="outer_block", outer_block_size=obs, outer_2d=o2d, rounding="stochastic",
                    seed=21, step=4, index_base=40)
    zd = torch.from_numpy(z0.copy()).cuda()
    out = fq.fp4_cast_transpose_grouped(dev(x), rows, g, residual=zd)
    zo = z0.copy()
    want = ref.nv_quantize_grouped(x, rows, two_level=tl, obs=obs, outer_2d=o2d, stochastic=True, seed=21, step=4,
                                   index_base=40, residual=zo)
    for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
        same(host(out[k], np.uint8).reshape(want[k].shape), want[k], "%d groups %s" % (len(rows), k))
    same(host(out["row_outer"], np.float32).ravel(), want["row_outer"], "row outer")
    if not o2d:
        same(host(out["col_outer"], np.float32).ravel(), want["col_outer"], "col outer")
    same(host(zd, np.float32), zo, "residual")


@pytest.mark.parametrize("o2d,staged", [(True, True), (True, False), (False, True), (False, False)])
def test_grouped_last_launch_holds_one_group(o2d, staged):
    """65 groups: the call's second launch holds the last group alone, at a
    nonzero first row, which the kernel form without the group bookkeeping
    (one group at row 0) must not take.  SR + error feedback, every buffer
    against the oracle."""
    rng = np.random.default_rng(31 + 2 * o2d + staged)
    rows = [int(v) for v in rng.choice([64, 128, 192], size=65)]
    C = 192
    x = rand_bf16(rng, (sum(rows), C), 0.02)
    z0 = (rng.standard_normal(x.shape) * 0.01).astype(np.float32)
    g = fq.make_cfg(format="nvfp4", two_level="outer_block", outer_block_size=64, outer_2d=o2d,
                    rounding="stochastic", seed=41, step=2, index_base=5)
    zd = torch.from_numpy(z0.copy()).cuda()
    out = fq.fp4_cast_transpose_grouped(dev(x), rows, g, residual=zd, staged=staged)
    zo = z0.copy()
    want = ref.nv_quantize_grouped(x, rows, two_level="outer", obs=64, outer_2d=o2d, stochastic=True, seed=41, step=2,
                                   index_base=5, residual=zo)
    for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
        same(host(out[k], np.uint8).reshape(want[k].shape), want[k], "65 groups %s" % k)
    same(host(out["row_outer"], np.float32).ravel(), want["row_outer"], "row outer")
    if not o2d:
        same(host(out["col_outer"], np.float32).ravel(), want["col_outer"], "col outer")
    same(host(zd, np.float32), zo, "residual")


def test_cast_transpose_1d_obs128_sr_16384x4096():
    """1D outer groups of 128 (1 x 128 along rows, 128 x 1 down columns; ALTO
    page, Technical design) at full size: AMD-FP4, SR, the 16384-token
    activation recipe on 4096 channels, every buffer against the oracle."""
    x = W.activations_16384x2880(cols=4096)
    g, o = cfgs("amdfp4", "outer", 128, False, True, seed=7, step=3)
    want = ref.nv_quantize(x, cols=True, want_y=False, **o)
    out = fq.fp4_cast_transpose(dev(x), g)
    for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
        same(host(out[k], np.uint8), want[k], "1D obs128 cast-transpose " + k)
    same(host(out["row_outer"], np.float32), want["row_outer"], "1D obs128 row outer")
    same(host(out["col_outer"], np.float32), want["col_outer"], "1D obs128 col outer")
