"""GPU parity at the stochastic-rounding decision boundaries and for
non-finite / overflowing values under error feedback.

Stochastic rounding ("fp4-train" README, Method): between grid neighbours
lo < hi an element rounds up iff u16 < frac * 2^16, frac = (t - lo) / (hi - lo),
with u16 the element's counter-based variate.  Random data almost never lands
next to that threshold, so these tests build inputs whose quotients t sit
exactly on it and one binary32 (or bf16) step either side, for every element's
own u16, in all seven grid intervals and in the subnormal range.  Every block
holds an anchor of magnitude 6, so its decoded inner scale is 1 and t is the
element's magnitude.  The device result must equal the oracle bit for bit and,
independently, the rule evaluated here in binary64 (where every quantity
involved is exact).

Sanitisation with error feedback (ALTO page, Op-level test coverage, read as:
the rule applies to the quantised sum x + r): NaN, +-inf and sums that overflow
binary32, with nonzero residuals, through the tile kernel and the rowwise
kernel.
"""
import zlib

import numpy as np
import pytest
import torch

import block_scaled_fp4_amax_amd as fq
from block_scaled_fp4_amax_amd import workloads as W
from oracle import ref

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fq.lib()


def host(t, dtype):
    torch.cuda.synchronize()
    return t.detach().cpu().contiguous().numpy().view(dtype)


def same(gpu, want, what):
    gpu, want = np.asarray(gpu), np.asarray(want)
    if want.dtype == np.float32:
        want = want.view(np.uint32)
        gpu = gpu.view(np.uint32)
    gpu = gpu.reshape(want.shape)
    bad = np.flatnonzero(gpu.ravel() != want.ravel())
    assert bad.size == 0, "%s: %d of %d differ; first at flat %d: gpu %s oracle %s" % (
        what, bad.size, want.size, bad[0], hex(int(gpu.ravel()[bad[0]])), hex(int(want.ravel()[bad[0]])))


def sr_rule(t, u):
    """E2M1 magnitude code of t >= 0 under stochastic rounding with variate u,
    evaluated in binary64 (t is a binary32 value: t - lo and the division by
    hi - lo in {0.5, 1, 2} are exact, and so is frac * 2^16)."""
    t = np.asarray(t, np.float64)
    lo = np.searchsorted(GRID, t, side="right") - 1
    lo = np.minimum(lo, 7)
    at_grid = GRID[lo] == t
    hi = GRID[np.minimum(lo + 1, 7)]
    width = np.where(lo < 7, hi - GRID[lo], 1.0)
    frac = (t - GRID[lo]) / width
    up = np.asarray(u, np.float64) < frac * 65536.0
    m = np.where(at_grid | (lo == 7), lo, lo + up.astype(np.int64))
    return np.where(t >= 6.0, 7, m)


def nibbles(codes, shape):
    c = np.asarray(codes, np.uint8).reshape(shape[0], shape[1] // 2)
    out = np.empty(shape, np.uint8)
    out[:, 0::2] = c & 0xF
    out[:, 1::2] = c >> 4
    return out


# ---------------------------------------------------------------- FP32 source, rowwise kernel
def _fp32_boundary_source(R, C, u, rng):
    """t at lo + u/65536 (hi - lo) for the element's own u and one binary32 step
    either side, grid points, values in (6, 6.375) that saturate under a scale of
    1, and subnormal / tiny values (placed where u is 0 or 1 as well as
    elsewhere); one anchor of magnitude 6 per 16-element block."""
    n = R * C
    uu = u.ravel().astype(np.float64)
    kind = rng.choice(5, n, p=[0.78, 0.05, 0.02, 0.10, 0.05])
    iv = rng.integers(0, 7, n)
    lo, hi = GRID[iv], GRID[iv + 1]
    t = np.empty(n, np.float32)
    t0 = (lo + uu / 65536.0 * (hi - lo)).astype(np.float32)           # exact in binary32
    assert np.all(t0.astype(np.float64) == lo + uu / 65536.0 * (hi - lo))
    step = rng.integers(-1, 2, n)
    tb = np.where(step < 0, np.nextafter(t0, np.float32(0)), np.where(step > 0, np.nextafter(t0, np.float32(7)), t0))
    t[:] = tb
    g = kind == 1
    t[g] = GRID[rng.integers(0, 8, g.sum())].astype(np.float32)
    s = kind == 2
    t[s] = rng.uniform(6.0, 6.37, s.sum()).astype(np.float32)
    sub = kind == 3
    t[sub] = (rng.integers(1, 1 << 23, sub.sum(), dtype=np.uint64).astype(np.uint32)).view(np.float32)
    tiny = kind == 4
    t[tiny] = np.float32(2.0) ** rng.integers(-140, -100, tiny.sum()).astype(np.float32)
    # subnormal quotients where the variate is 0 or 1: only u == 0 rounds up
    low_u = np.flatnonzero(uu <= 1)
    t[low_u] = (rng.integers(1, 1 << 23, low_u.size, dtype=np.uint64).astype(np.uint32)).view(np.float32)
    t = t.reshape(R, C)
    t[:, ::16] = 6.0                                          # anchors: block scale 1
    sign = rng.integers(0, 2, (R, C)).astype(bool)
    return np.where(sign, -t, t).astype(np.float32), low_u


@pytest.mark.parametrize("index_base", [0, 13])
def test_sr_boundaries_fp32_rowwise(index_base):
    R, C = 512, 1024
    seed, step = 7, 3
    rng = np.random.default_rng(100 + index_base)
    u = ref.sr_u16_array(seed, step, index_base, R * C).reshape(R, C)
    x, low_u = _fp32_boundary_source(R, C, u, rng)
    assert np.sum(u.ravel()[low_u] == 0) > 0, "no element with u16 == 0 in the sample"
    cfg = fq.make_cfg(format="nvfp4", rounding="stochastic", seed=seed, step=step, index_base=index_base)
    out = fq.fp4_quantize(torch.from_numpy(x).cuda(), cfg)
    codes, scales = host(out["codes"], np.uint8), host(out["scales"], np.uint8)
    want = ref.nv_quantize(x, stochastic=True, seed=seed, step=step, index_base=index_base)
    same(scales, want["row_scales"], "scales")
    same(codes, want["row_codes"], "codes")
    # the rule, independently of the oracle
    assert np.all(scales == 0x38), "every block's decoded scale is 1"
    m = nibbles(codes, (R, C))
    same(m & 7, sr_rule(np.abs(x), u).astype(np.uint8), "magnitude codes vs the rounding rule")
    same(m >> 3, np.signbit(x).astype(np.uint8), "sign bits")


# ---------------------------------------------------------------- bf16 source, tile kernel
def _bf16_boundary_source(R, C, u, rng, tile_anchor):
    """bf16 values next to each element's threshold: in [lo, hi) with n bf16
    steps, the grid value k steps above lo has threshold k * 65536 / n, so the
    two values around u (k = floor(u n / 65536) and k + 1) sit on either side
    of it, exactly on it where u is a multiple of 65536 / n.  In [0, 0.5) the
    threshold of t is t * 2^17: t = u / 2^17 is exact for small u.  Anchors of
    magnitude 6 on the 16 x 16 diagonals give every row block and every column
    block the scale 1; with tile_anchor a value of 2688 at each 64 x 64 tile's
    (0, 0) makes its 2D outer scale 1."""
    n_el = R * C
    uu = u.ravel().astype(np.int64)
    iv = rng.integers(0, 7, n_el)
    t = np.empty(n_el, np.float64)
    steps = {1: 128, 2: 64, 3: 64, 4: 64, 5: 64, 6: 64}
    for k, n in steps.items():
        sel = iv == k
        kk = (uu[sel] * n) // 65536 + rng.integers(0, 2, sel.sum())
        t[sel] = GRID[k] + kk * (GRID[k + 1] - GRID[k]) / n
    sel = iv == 0
    t[sel] = uu[sel] / 131072.0 * np.exp2(rng.integers(-1, 2, sel.sum()) * 0.0)
    small = sel & (uu < 256)
    t[small] = uu[small] / 131072.0 + rng.integers(-1, 2, small.sum()) * 2.0 ** -25
    t = np.abs(t)
    tb = W.to_bf16(t.astype(np.float32)).reshape(R, C)
    # subnormal bf16 where u <= 1
    low = (u <= 1)
    tb[low] = rng.integers(1, 0x80, low.sum()).astype(np.uint16)
    i = np.arange(R)[:, None]
    j = np.arange(C)[None, :]
    tb[(i % 16) == (j % 16)] = W.to_bf16(np.float32([6.0]))[0]
    if tile_anchor:
        tb[::64, ::64] = W.to_bf16(np.float32([2688.0]))[0]
    sign = rng.integers(0, 2, (R, C)).astype(np.uint16) << 15
    return tb | sign


@pytest.mark.parametrize("mode", ["none", "outer2d"])
def test_sr_boundaries_bf16_cast_transpose(mode):
    R, C = 512, 1024
    seed, step, ib = 5, 2, 0
    rng = np.random.default_rng(7 if mode == "none" else 8)
    u = ref.sr_u16_array(seed, step, ib, R * C).reshape(R, C)
    x = _bf16_boundary_source(R, C, u, rng, tile_anchor=(mode == "outer2d"))
    if mode == "none":
        cfg = fq.make_cfg(format="nvfp4", rounding="stochastic", seed=seed, step=step)
        kw = {}
    else:
        cfg = fq.make_cfg(format="nvfp4", two_level="outer_block", outer_block_size=64, outer_2d=True,
                          rounding="stochastic", seed=seed, step=step)
        kw = dict(two_level="outer", obs=64, outer_2d=True)
    out = fq.fp4_cast_transpose(torch.from_numpy(x.view(np.int16)).cuda(), cfg)
    want = ref.nv_quantize(x, stochastic=True, seed=seed, step=step, cols=True, want_y=False, **kw)
    for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
        same(host(out[k], np.uint8), want[k], "%s %s" % (mode, k))
    if mode == "outer2d":
        o = host(out["row_outer"], np.float32)
        assert np.all(o == 1.0), "every 64 x 64 tile's outer scale is 1"
        same(o, want["row_outer"], "outer")
    # the rule on every element whose row block and column block have scale 1
    t = np.abs(W.from_bf16(x)).astype(np.float64)
    m_row = nibbles(host(out["row_codes"], np.uint8), (R, C))
    m_col = nibbles(host(out["col_codes"], np.uint8), (C, R)).T
    rs = np.repeat(host(out["row_scales"], np.uint8).reshape(R, C // 16), 16, axis=1)
    cs = np.repeat(host(out["col_scales"], np.uint8).reshape(C, R // 16), 16, axis=1).T
    ok = (rs == 0x38) & (cs == 0x38)
    assert ok.mean() > 0.99
    rule = sr_rule(t, u).astype(np.uint8)
    same((m_row & 7)[ok], rule[ok], "%s row codes vs the rounding rule" % mode)
    same((m_col & 7)[ok], rule[ok], "%s col codes vs the rounding rule" % mode)
    # exact-threshold hits were exercised: t * 2^16 / width == u for some elements
    lo = np.searchsorted(GRID, t, side="right") - 1
    lo = np.minimum(lo, 6)
    frac = (t - GRID[lo]) / (GRID[lo + 1] - GRID[lo])
    exact_hit = (frac * 65536.0 == u) & (t > 0) & (t < 6) & ok
    assert exact_hit.sum() > 100


# ---------------------------------------------------------------- error feedback with non-finite values
EDGE = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x0040, 0x7F7F, 0xFF7F, 0x7F80, 0xFF80, 0x7FC0, 0xFFC1,
                 0x3F80, 0xBF80, 0x4013, 0x7F62, 0xFF62], np.uint16)


def _edge_inputs(R, C, seed):
    rng = np.random.default_rng(seed)
    x = rng.choice(EDGE, size=(R, C)).astype(np.uint16)
    x[: R // 2, : C // 2] = W.to_bf16(rng.standard_normal((R // 2, C // 2)).astype(np.float32))
    z = (rng.standard_normal((R, C)) * 0.25).astype(np.float32)
    big = (x & 0x7FFF) == 0x7F62                       # |x| = 3.0e38: these sums overflow
    z[big] = np.where(x[big] >> 15 == 1, np.float32(-9e37), np.float32(9e37))
    return x, z


EF_CT_CASES = [
    # fmt, two_level, obs, outer_2d, sr
    ("nvfp4", "none", 0, False, True),
    ("nvfp4", "tensorwise", 0, False, False),
    ("amdfp4", "tensorwise", 0, False, True),
    ("nvfp4", "outer", 64, True, True),
    ("nvfp4", "outer", 64, True, False),
    ("amdfp4", "outer", 64, False, True),
    ("nvfp4", "outer", 32, False, False),
]
FMT = {"nvfp4": "e4m3", "amdfp4": "ue5m3"}


@pytest.mark.parametrize("case", EF_CT_CASES, ids=lambda c: "-".join(str(v) for v in c))
def test_error_feedback_edge_values_cast_transpose(case):
    fmt, tl, obs, o2d, sr = case
    R, C = 128, 192
    x, z0 = _edge_inputs(R, C, zlib.crc32(repr(case).encode()))
    gtl = {"none": "none", "tensorwise": "tensorwise", "outer": "outer_block"}[tl]
    cfg = fq.make_cfg(format=fmt, two_level=gtl, outer_block_size=obs, outer_2d=o2d,
                      rounding="stochastic" if sr else "rne", seed=4, step=6)
    zo = z0.copy()
    want = ref.nv_quantize(x, scale_fmt=FMT[fmt], two_level=tl, obs=obs, outer_2d=o2d, stochastic=sr, seed=4, step=6,
                           residual=zo, cols=True, want_y=False)
    zd = torch.from_numpy(z0.copy()).cuda()
    out = fq.fp4_cast_transpose(torch.from_numpy(x.view(np.int16)).cuda(), cfg, residual=zd)
    for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
        same(host(out[k], np.uint8), want[k], k)
    for k in ("row_outer", "col_outer"):
        if k in want:
            same(host(out[k], np.float32), want[k], k)
    same(host(zd, np.float32), zo, "residual")
    assert np.all(np.isfinite(zo))


@pytest.mark.parametrize("case", EF_CT_CASES + [("nvfp4", "outer", 128, False, True)],
                         ids=lambda c: "-".join(str(v) for v in c))
def test_error_feedback_edge_values_qdq(case):
    fmt, tl, obs, o2d, sr = case
    R, C = 128, 256
    x, z0 = _edge_inputs(R, C, zlib.crc32(repr(case).encode()) + 1)
    gtl = {"none": "none", "tensorwise": "tensorwise", "outer": "outer_block"}[tl]
    cfg = fq.make_cfg(format=fmt, two_level=gtl, outer_block_size=obs, outer_2d=o2d,
                      rounding="stochastic" if sr else "rne", seed=4, step=6)
    zo = z0.copy()
    want = ref.nv_quantize(x, scale_fmt=FMT[fmt], two_level=tl, obs=obs, outer_2d=o2d, stochastic=sr, seed=4, step=6,
                           residual=zo)
    zd = torch.from_numpy(z0.copy()).cuda()
    out = fq.fp4_qdq(torch.from_numpy(x.view(np.int16)).cuda(), cfg, residual=zd, with_codes=True)
    same(host(out["y"].view(torch.int16), np.uint16), want["row_y"], "y")
    same(host(out["codes"], np.uint8), want["row_codes"], "codes")
    same(host(out["scales"], np.uint8), want["row_scales"], "scales")
    if "row_outer" in want:
        same(host(out["outer"], np.float32), want["row_outer"], "outer")
    same(host(zd, np.float32), zo, "residual")
