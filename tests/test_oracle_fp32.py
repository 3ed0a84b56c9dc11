"""Pins of the oracle's binary32 source and binary32 targets ("fp4-train"
README, Requirements and limits: float32 or bfloat16 input; "MXFP4 weight QAT
recipes", Correctness: fake-quant on bf16 and fp32, dequantise to bf16 and fp32
targets, fp32 raw-bit fuzz).

Independent references: the exact-rational model (oracle/exact.py, which shares
no code with the C oracle) on raw binary32 bit patterns and on the edge values
of each format; the bf16 source path, pinned elsewhere, for binary32 sources
that hold bf16 values; closed forms for MXFP4 outputs (exact in bf16, so the
binary32 target is the bf16 one widened)."""
import zlib

import numpy as np
import pytest

from oracle import exact, ref

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

KEYS = ["row_codes", "row_scales", "row_outer", "row_y", "col_codes", "col_scales", "col_outer", "col_y"]


def _bits(a):
    a = np.asarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def _compare(c_out, e_out, keys):
    for k in keys:
        if k not in e_out:
            continue
        a, b = np.asarray(c_out[k]), np.asarray(e_out[k])
        if b.dtype == np.float32 or a.dtype == np.float32:
            a, b = a.astype(np.float32).view(np.uint32), b.astype(np.float32).view(np.uint32)
        np.testing.assert_array_equal(a.reshape(b.shape), b, err_msg=k)


def _widen(bf):
    return (np.asarray(bf, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _fp32_source(rng, shape):
    """Full-mantissa binary32 values: lognormal row ranges, an outlier row, a
    tiny column, signed zeros, and raw bit patterns (subnormals, huge values)."""
    R, C = shape
    x = (rng.standard_normal(shape) * np.exp(2 * rng.standard_normal((R, 1)))).astype(np.float32)
    x[rng.integers(0, R), :] *= np.float32(300)
    x[:, rng.integers(0, C)] *= np.float32(1e-3)
    x.ravel()[rng.integers(0, R * C, 5)] = 0.0
    x.ravel()[rng.integers(0, R * C, 3)] = -0.0
    raw = rng.integers(0, 1 << 32, 12, dtype=np.uint64).astype(np.uint32)
    raw &= np.uint32(0xBFFFFFFF)            # exponent below 0x80: finite, magnitudes < 2
    x.ravel()[rng.integers(0, R * C, 12)] = raw.view(np.float32)
    sub = rng.integers(1, 1 << 23, 4, dtype=np.uint64).astype(np.uint32)
    x.ravel()[rng.integers(0, R * C, 4)] = sub.view(np.float32)      # binary32 subnormals
    return x


MODES = [
    # (scale_fmt, two_level, obs, outer_2d, stochastic, ef, cols, shape)
    ("e4m3", "none", 0, False, False, False, True, (32, 48)),
    ("e4m3", "tensorwise", 0, False, False, False, True, (32, 32)),
    ("e4m3", "outer", 32, False, False, False, True, (32, 64)),
    ("ue5m3", "outer", 16, True, True, False, True, (32, 32)),
    ("e4m3", "none", 0, False, True, True, False, (16, 64)),
    ("ue5m3", "tensorwise", 0, False, False, True, False, (16, 32)),
    ("e4m3", "outer", 32, False, True, True, False, (16, 64)),
]


@pytest.mark.parametrize("y32", [False, True], ids=["y_bf16", "y_fp32"])
@pytest.mark.parametrize("mode", MODES, ids=lambda m: "-".join(str(v) for v in m[:7]))
def test_nv_fp32_source_matches_exact_model(mode, y32):
    sfmt, tl, obs, o2d, sr, ef, cols, shape = mode
    rng = np.random.default_rng(zlib.crc32(repr(mode).encode()))
    R, C = shape
    x = _fp32_source(rng, shape)
    resid = (rng.standard_normal(shape) * 0.01).astype(np.float32) if ef else None
    kw = dict(scale_fmt=sfmt, two_level=tl, obs=obs, outer_2d=o2d, stochastic=sr, seed=9, step=4, index_base=77)
    res_c = None if resid is None else resid.copy()
    c_out = ref.nv_quantize(x, residual=res_c, cols=cols, y_dtype="fp32" if y32 else "bf16", **kw)
    u = ref.sr_u16_array(9, 4, 77, R * C).reshape(R, C) if sr else None
    e_out = exact.nv_quantize(x.view(np.uint32), scale_fmt=sfmt, two_level=tl, obs=obs, outer_2d=o2d,
                              stochastic=sr, u16=u, residual=resid, cols=cols, y_f32=y32)
    _compare(c_out, e_out, KEYS)
    if ef:
        np.testing.assert_array_equal(res_c.view(np.uint32), e_out["residual"].view(np.uint32))


def test_nv_fp32_edge_values_match_exact_model():
    # signed zeros, the smallest and largest subnormals, the largest finite
    # binary32 (beyond bf16's), +-inf and NaN (sanitised), values on either side
    # of the bf16 range's top, 1 and a binary32 ulp either side of it
    vals = np.array([0x00000000, 0x80000000, 0x00000001, 0x807FFFFF, 0x00400000, 0x7F7FFFFF, 0xFF7FFFFF,
                     0x7F800000, 0xFF800000, 0x7FC00001, 0x7F7F0000, 0x7F7F8000, 0x3F800000, 0x3F800001,
                     0x3F7FFFFF, 0x40C00001], np.uint32)
    rng = np.random.default_rng(5)
    for tl, obs, o2d in [("none", 0, False), ("tensorwise", 0, False), ("outer", 16, True), ("outer", 16, False)]:
        for sfmt in ("e4m3", "ue5m3"):
            xb = rng.choice(vals, size=(16, 32)).astype(np.uint32)
            xb[:, 16:] = rng.choice(vals[:5], size=(16, 16))          # a block of tiny / zero values
            x = xb.view(np.float32)
            for y32 in (False, True):
                c_out = ref.nv_quantize(x, scale_fmt=sfmt, two_level=tl, obs=obs, outer_2d=o2d, cols=True,
                                        y_dtype="fp32" if y32 else "bf16")
                e_out = exact.nv_quantize(xb, scale_fmt=sfmt, two_level=tl, obs=obs, outer_2d=o2d, cols=True,
                                          y_f32=y32)
                _compare(c_out, e_out, KEYS)


@pytest.mark.parametrize("tl,obs,o2d,sr,ef", [("none", 0, False, False, False), ("tensorwise", 0, False, True, True),
                                               ("outer", 32, False, True, False), ("outer", 16, True, False, True)])
def test_nv_fp32_source_of_bf16_values_equals_bf16_source(tl, obs, o2d, sr, ef):
    rng = np.random.default_rng(17)
    xb = ref.f32_to_bf16((rng.standard_normal((64, 64)) * 0.05).astype(np.float32))
    xb[3, :7] = [0x0000, 0x8000, 0x0001, 0x7F80, 0xFF80, 0x7FC0, 0x7F7F]
    kw = dict(two_level=tl, obs=obs, outer_2d=o2d, stochastic=sr, seed=3, step=1, cols=True)
    r0 = (rng.standard_normal((64, 64)) * 1e-3).astype(np.float32) if ef else None
    r1 = None if r0 is None else r0.copy()
    a = ref.nv_quantize(xb, residual=r0, **kw)
    b = ref.nv_quantize(_widen(xb), residual=r1, **kw)
    for k in a:
        np.testing.assert_array_equal(_bits(a[k]), _bits(b[k]), err_msg=k)
    if ef:
        np.testing.assert_array_equal(r0.view(np.uint32), r1.view(np.uint32))


def test_nv_fp32_target_rounds_to_the_bf16_target():
    """The bf16 output is the RNE of the binary32 output; without an outer
    scale the two are equal (G[m] * d has at most 5 significant bits)."""
    rng = np.random.default_rng(23)
    x = _fp32_source(rng, (32, 64))
    for tl, obs, o2d in [("none", 0, False), ("tensorwise", 0, False), ("outer", 32, False), ("outer", 16, True)]:
        y16 = ref.nv_quantize(x, two_level=tl, obs=obs, outer_2d=o2d)["row_y"]
        y32 = ref.nv_quantize(x, two_level=tl, obs=obs, outer_2d=o2d, y_dtype="fp32")["row_y"]
        np.testing.assert_array_equal(ref.f32_to_bf16(y32), y16)
        if tl == "none":
            np.testing.assert_array_equal(y32.view(np.uint32), _widen(y16).view(np.uint32))


def test_nv_fp32_dequantize_reproduces_the_qdq_target():
    rng = np.random.default_rng(29)
    x = _fp32_source(rng, (32, 64))
    for tl, obs, o2d, kind in [("none", 0, False, "none"), ("tensorwise", 0, False, "tensorwise"),
                               ("outer", 32, False, "1d"), ("outer", 16, True, "2d")]:
        q = ref.nv_quantize(x, two_level=tl, obs=obs, outer_2d=o2d, y_dtype="fp32")
        y = ref.nv_dequantize(q["row_codes"], q["row_scales"], q.get("row_outer"), 32, 64, outer_kind=kind, obs=obs,
                              y_dtype="fp32")
        np.testing.assert_array_equal(y.view(np.uint32), q["row_y"].view(np.uint32))


def _mx_fuzz(rng, R, C):
    """Raw binary32 bit patterns in blocks of one binade range each, plus
    blocks of full-range raw bits (NaN / inf / subnormal patterns included)."""
    x = np.zeros((R, C), np.uint32)
    for i in range(R):
        for j0 in range(0, C, 32):
            kind = (i * (C // 32) + j0 // 32) % 4
            raw = rng.integers(0, 1 << 32, 32, dtype=np.uint64).astype(np.uint32)
            if kind == 0:
                x[i, j0:j0 + 32] = raw                                   # anything, incl. NaN / inf
            else:
                e = int(rng.integers(1, 250)) if kind != 3 else 0        # kind 3: subnormals
                span = np.uint32(int(rng.integers(0, 4)) << 23)
                x[i, j0:j0 + 32] = (raw & np.uint32(0x807FFFFF)) | np.uint32(e << 23)
                x[i, j0:j0 + 32] += (raw % np.uint32(4)) * np.uint32(1 << 23) & span
    return x


def test_mx_fp32_raw_bit_fuzz_matches_exact_model():
    rng = np.random.default_rng(31)
    xb = _mx_fuzz(rng, 16, 256)
    xb[0, :32] = [0x00000000, 0x80000000, 0x00000001, 0x80000003, 0x00400000, 0x00800000, 0x7F7FFFFF,
                  0x7F3FFFFF, 0x7F400000, 0x7F400001, 0x40C00000, 0x40C00001, 0x40BFFFFF, 0x3E800000,
                  0x3E800001, 0x3E7FFFFF, 0x3F400000, 0x3FA00000, 0x3FE00000, 0x40200000, 0x40600000,
                  0x40A00000, 0x3F400001, 0x3FA00001, 0xBFE00001, 0x40200001, 0xC0600001, 0x40A00001,
                  0x3F3FFFFF, 0x3F9FFFFF, 0x3FDFFFFF, 0x405FFFFF]
    x = xb.view(np.float32)
    for y32 in (False, True):
        c, s, y = ref.mx_qdq(x, y_dtype="fp32" if y32 else "bf16")
        ce, se, ye = exact.mx_qdq(xb, y_f32=y32)
        np.testing.assert_array_equal(c, ce)
        np.testing.assert_array_equal(s, se)
        np.testing.assert_array_equal(_bits(y), _bits(ye.astype(np.float32) if y32 else ye))


def test_mx_fp32_target_is_the_bf16_target_widened():
    """Every projected value +-G[m] 2^k (k in [-126, 125]) is exact in bf16, so
    the binary32 target equals the bf16 one widened, for both sources."""
    rng = np.random.default_rng(37)
    xb = _mx_fuzz(rng, 32, 512)
    x = xb.view(np.float32)
    c16, s16, y16 = ref.mx_qdq(x)
    c32, s32, y32 = ref.mx_qdq(x, y_dtype="fp32")
    np.testing.assert_array_equal(c16, c32)
    np.testing.assert_array_equal(s16, s32)
    np.testing.assert_array_equal(y32.view(np.uint32), _widen(y16).view(np.uint32))
    np.testing.assert_array_equal(ref.mx_dequantize(c32, s32, 32, 512, y_dtype="fp32").view(np.uint32),
                                  y32.view(np.uint32))


def test_mx_fp32_source_of_bf16_values_equals_bf16_source():
    xb = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
    a = ref.mx_qdq(xb)
    b = ref.mx_qdq(_widen(xb))
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


def test_mx_fp32_projection_is_idempotent():
    rng = np.random.default_rng(41)
    x = _mx_fuzz(rng, 32, 256).view(np.float32)
    _, _, y = ref.mx_qdq(x, y_dtype="fp32")
    fin = np.isfinite(y).reshape(32, -1, 32).all(axis=2)
    _, _, y2 = ref.mx_qdq(y, y_dtype="fp32")
    blocks = np.repeat(fin, 32, axis=1)
    np.testing.assert_array_equal(y2.view(np.uint32)[blocks], y.view(np.uint32)[blocks])
