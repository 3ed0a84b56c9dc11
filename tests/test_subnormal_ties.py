"""Outer normalisation at exact ties of the binary32 subnormal grid.

The kernels normalise by an outer scale as RN32(v * RN64(1 / s)) and form the
outer scale as RN32(amax * RN64(1 / den)).  Such a product equals the correctly
rounded quotient unless that quotient is an exact tie on the subnormal grid,
so every subnormal result is divided again in binary32.

- Normalisation: with s = 49 * 2^18, RN64(1 / s) lies 0.72 of a half-ulp below
  1 / s, so for v = 3 * 2^-150 * s = 147 * 2^-132 (a bf16 value) the product
  rounds to 2^-149 where v / s = 3 * 2^-150 rounds to 2^-148 (even).  The
  difference reaches the codes when the block's inner scale is d = 2 (the
  block holds 12 s = 147 * 2^20, normalised to 12): t = RN32(v_n / 2) is
  2^-149 for the correct v_n and 0 (a tie at 2^-150) for the other, and under
  stochastic rounding a nonzero t rounds up to code 1 when its variate is 0.
  index_base puts a zero variate on one such element.  The group maximum
  s * den = 1029 * 2^25 is not a bf16 value: the computed scales come through
  the binary32-source and error-feedback paths, and bf16 sources get s as a
  caller-supplied outer scale.
- Outer scale: a maximum of 63 * 2^-143 (NVFP4, den = 2688 = 21 * 2^7; AMD-FP4
  63 * 2^-135, den = 21 * 2^15) gives amax / den = 3 * 2^-150, a tie, which
  rounds to 2^-148.  Here the product is right for every tie (the CPU test
  below checks all of them), so this block only pins the tie end to end.

Each 64 x 64 block is symmetric, so the columnwise groups see the same ties
as the rowwise ones.  Every output buffer is compared byte for byte with the
oracle ("NVFP4 / AMD-FP4 outer-block (two-level) scaling for FP4 training",
Technical design: the per-block scale, the normalisation by it; "fp4-train"
README, Method: the stochastic rounding rule)."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_amax_amd as fq
from block_scaled_fp4_amax_amd import workloads as W
from oracle import ref

SEED, STEP = 0x5EED_71E5, 11
DEN = {"nvfp4": 2688.0, "amdfp4": 688128.0}
SFMT = {"nvfp4": "e4m3", "amdfp4": "ue5m3"}
S_NORM = np.float32(49 * 2 ** 18)
B_NORM = np.float32(12 * 49 * 2 ** 18)   # normalised to 12: inner scale 2
ZERO_AT = (3, 20)   # the tie element that gets a zero variate (row, column)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fq.lib()


def norm_tie_block(fmt, n=64):
    """Symmetric: s * den on the diagonal (each 64-group's maximum), 12 s at
    (i, i ^ 16), +-3 * 2^-150 * s over the rest of that 16-block."""
    A = np.float32(S_NORM * np.float32(DEN[fmt]))
    T = np.float32(float(S_NORM) * 3 * 2.0 ** -150)   # exact: 147 * 2^-132
    M = np.zeros((n, n), np.float32)
    for i in range(n):
        b = (i ^ 16) & ~15
        for j in range(b, b + 16):
            M[i, j] = T if (i + j) % 2 == 0 else -T
        M[i, i ^ 16] = B_NORM
        M[i, i] = A
    assert (M == M.T).all()
    return M


def outer_tie_block(fmt, n=64, seed=1):
    """Symmetric: 63 * 2^-(143 or 135) on the diagonal, smaller multiples of
    2^-149 elsewhere (their quotients by 2^-148 are exact halves)."""
    top = np.float32(63 * 2.0 ** (-143 if fmt == "nvfp4" else -135))
    rng = np.random.default_rng(seed)
    k = rng.integers(-40, 40, size=(n, n)).astype(np.float32) * np.float32(2.0 ** -149)
    M = np.triu(k, 1)
    M = M + M.T
    np.fill_diagonal(M, top)
    assert (M == M.T).all()
    return M


def tie_matrix(fmt):
    """128 x 128: the normalisation ties in the top-left 64 x 64 block, the
    outer-scale ties in the bottom-right one, zeros elsewhere."""
    X = np.zeros((128, 128), np.float32)
    X[:64, :64] = norm_tie_block(fmt)
    X[64:, 64:] = outer_tie_block(fmt)
    return X


def zero_variate_base(cols):
    """index_base that gives element ZERO_AT a zero 16-bit variate."""
    off = ZERO_AT[0] * cols + ZERO_AT[1]
    lo = 1 << 20
    u = ref.sr_u16_array(SEED, STEP, lo, 1 << 22)
    hits = np.flatnonzero(u == 0)
    assert hits.size, "no zero variate in the searched range"
    base = lo + int(hits[0]) - off
    assert ref.sr_u16(SEED, STEP, base + off) == 0
    return base


def test_cases_are_discriminating():
    """(CPU) Pins the construction: the normalisation tie comes out of the
    unchecked binary64 product on the other side, and the difference survives
    into t = v_n / 2; every outer-scale tie of both formats comes out right."""
    T = np.float32(float(S_NORM) * 3 * 2.0 ** -150)   # exact: 147 * 2^-132
    assert T == np.float32(147 * 2.0 ** -132) and ref.f32_to_bf16(np.array([T]))[0] != 0
    assert ref.bf16_to_f32(ref.f32_to_bf16(np.array([T])))[0] == T          # a bf16 value
    exact = ref.div_f32(np.array([T]), np.array([S_NORM]))[0]
    prod = np.float32(np.float64(T) * (1.0 / np.float64(S_NORM)))
    assert exact == np.float32(2.0 ** -148) and prod == np.float32(2.0 ** -149)
    d = np.float32(2.0)
    assert ref.div_f32(np.array([exact]), np.array([d]))[0] == np.float32(2.0 ** -149)
    assert ref.div_f32(np.array([prod]), np.array([d]))[0] == 0.0
    for fmt, den in DEN.items():
        A = norm_tie_block(fmt)[0, 0]
        assert ref.div_f32(np.array([A]), np.array([den], np.float32))[0] == S_NORM
        assert ref.div_f32(np.array([B_NORM]), np.array([S_NORM]))[0] == 12.0
        assert ref.bf16_to_f32(ref.f32_to_bf16(np.array([B_NORM])))[0] == B_NORM   # a bf16 value
        # every tie amax / den = M 2^-150 (M odd, amax = 21 M 2^e a binary32)
        M = np.arange(1, (1 << 24) // 21 + 1, 2, dtype=np.int64)
        e = -143 if fmt == "nvfp4" else -135
        amax = ((21 * M).astype(np.float64) * 2.0 ** e).astype(np.float32)
        assert (amax.astype(np.float64) == (21 * M).astype(np.float64) * 2.0 ** e).all()
        q = ref.div_f32(amax, np.full(amax.shape, den, np.float32))
        p = (amax.astype(np.float64) * (1.0 / den)).astype(np.float32)
        assert (q == p).all(), fmt
        top = outer_tie_block(fmt)[0, 0]
        assert ref.div_f32(np.array([top]), np.array([den], np.float32))[0] == np.float32(2.0 ** -148)
    X = norm_tie_block("nvfp4")
    assert abs(X[ZERO_AT]) == T and X[ZERO_AT[0], ZERO_AT[0] ^ 16] == B_NORM


def _same(gpu, want, what):
    gpu, want = np.asarray(gpu), np.asarray(want)
    if want.dtype == np.float32:
        want, gpu = want.view(np.uint32), gpu.view(np.uint32)
    gpu = gpu.reshape(want.shape)
    bad = np.flatnonzero(gpu.ravel() != want.ravel())
    assert bad.size == 0, "%s: %d of %d differ; first at flat %d: gpu %s oracle %s" % (
        what, bad.size, want.size, bad[0], hex(int(gpu.ravel()[bad[0]])), hex(int(want.ravel()[bad[0]])))


def _host(t, dtype):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.detach().cpu().contiguous().numpy().view(dtype)


def _cfg(fmt, obs, outer_2d, base):
    return fq.make_cfg(format=fmt, two_level="outer_block", outer_block_size=obs, outer_2d=outer_2d,
                       rounding="stochastic", seed=SEED, step=STEP, index_base=base)


def _oracle_kw(fmt, obs, outer_2d, base):
    return dict(scale_fmt=SFMT[fmt], two_level="outer", obs=obs, outer_2d=outer_2d, stochastic=True, seed=SEED,
                step=STEP, index_base=base)


@pytest.mark.gpu
@pytest.mark.parametrize("fmt", ["nvfp4", "amdfp4"])
@pytest.mark.parametrize("obs", [64, 128])
@pytest.mark.parametrize("op", ["quantize", "qdq"])
def test_rowwise_fp32_source(dev, fmt, obs, op):
    """Rowwise kernel, binary32 source, 1D outer groups."""
    X = tie_matrix(fmt)
    base = zero_variate_base(X.shape[1])
    want = ref.nv_quantize(X, want_y=op == "qdq", y_dtype="fp32", **_oracle_kw(fmt, obs, False, base))
    g = _cfg(fmt, obs, False, base)
    xd = torch.from_numpy(X).cuda()
    if op == "qdq":
        out = fq.fp4_qdq(xd, g, with_codes=True, y_dtype=torch.float32)
        _same(_host(out["y"], np.float32), want["row_y"], "y")
    else:
        out = fq.fp4_quantize(xd, g)
    _same(_host(out["codes"], np.uint8), want["row_codes"], "codes")
    _same(_host(out["scales"], np.uint8), want["row_scales"], "scales")
    _same(_host(out["outer"], np.float32), want["row_outer"], "outer")


def _split_bf16_and_residual(X):
    """x (bf16 bits) and a residual with x + r = X exactly: bf16-exact entries
    go in x, the rest in the residual."""
    xb = W.to_bf16(X)
    back = ref.bf16_to_f32(xb)
    exact = back == X
    xb = np.where(exact, xb, np.uint16(0)).astype(np.uint16)
    r = np.where(exact, np.float32(0), X).astype(np.float32)
    return xb, r


@pytest.mark.gpu
@pytest.mark.parametrize("fmt", ["nvfp4", "amdfp4"])
@pytest.mark.parametrize("mode", ["1d64", "1d128", "2d"])
@pytest.mark.parametrize("staged", [True, False])
def test_cast_transpose_with_residual(dev, fmt, mode, staged):
    """Tile kernel (both directions), error feedback carrying the values that
    bf16 cannot hold; staged and direct stores."""
    X = tie_matrix(fmt)
    xb, r = _split_bf16_and_residual(X)
    obs = 128 if mode == "1d128" else 64
    o2d = mode == "2d"
    base = zero_variate_base(X.shape[1])
    zo = r.copy()
    want = ref.nv_quantize(xb, residual=zo, cols=True, want_y=False, **_oracle_kw(fmt, obs, o2d, base))
    zd = torch.from_numpy(r.copy()).cuda()
    out = fq.fp4_cast_transpose(torch.from_numpy(xb.view(np.int16)).cuda(), _cfg(fmt, obs, o2d, base), residual=zd,
                                staged=staged)
    for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
        _same(_host(out[k], np.uint8), want[k], k)
    for k in ("row_outer", "col_outer"):
        if k in want:
            _same(_host(out[k], np.float32), want[k], k)
    _same(_host(zd, np.float32), zo, "residual")


@pytest.mark.gpu
@pytest.mark.parametrize("fmt", ["nvfp4", "amdfp4"])
def test_grouped_2d(dev, fmt):
    """Grouped launch (two groups of the tie matrix), 2D outer tiles, error
    feedback."""
    X = np.concatenate([tie_matrix(fmt), tie_matrix(fmt)[::-1, ::-1].copy()])
    xb, r = _split_bf16_and_residual(X)
    rows = [128, 128]
    base = zero_variate_base(X.shape[1])
    zo = r.copy()
    want = ref.nv_quantize_grouped(xb, rows, residual=zo, **_oracle_kw(fmt, 64, True, base))
    zd = torch.from_numpy(r.copy()).cuda()
    out = fq.fp4_cast_transpose_grouped(torch.from_numpy(xb.view(np.int16)).cuda(), rows,
                                        _cfg(fmt, 64, True, base), residual=zd)
    for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
        _same(_host(out[k], np.uint8).reshape(want[k].shape), want[k], k)
    _same(_host(out["row_outer"], np.float32).ravel(), want["row_outer"].ravel(), "row_outer")
    _same(_host(zd, np.float32), zo, "residual")


def _given_outer(shape_rows, shape_cols, rows_in_block, cols_in_block):
    """Outer scales: s where the group lies in the normalisation tie block,
    1 elsewhere."""
    o = np.ones((shape_rows, shape_cols), np.float32)
    o[rows_in_block, cols_in_block] = S_NORM
    return o


@pytest.mark.gpu
@pytest.mark.parametrize("fmt", ["nvfp4", "amdfp4"])
@pytest.mark.parametrize("mode", ["1d64", "2d"])
@pytest.mark.parametrize("op", ["quantize", "ct"])
def test_bf16_with_given_outer(dev, fmt, mode, op):
    """bf16 source, no residual, outer scales supplied by the caller: the
    normalisation tie through the rowwise kernel and both directions of the
    tile kernel."""
    X = np.zeros((128, 128), np.float32)
    X[:64, :64] = norm_tie_block(fmt)
    np.fill_diagonal(X, 0.0)                        # s * den is not a bf16 value; s is given
    xb = W.to_bf16(X)
    assert (ref.bf16_to_f32(xb) == X).all()
    o2d = mode == "2d"
    if o2d:
        row_o, col_o = _given_outer(2, 2, 0, 0), None
    else:
        row_o = _given_outer(128, 2, slice(0, 64), 0)   # [rows, cols / 64]
        col_o = _given_outer(128, 2, slice(0, 64), 0)   # [cols, rows / 64]
    base = zero_variate_base(X.shape[1])
    kw = _oracle_kw(fmt, 64, o2d, base)
    g = _cfg(fmt, 64, o2d, base)
    g.outer_mode = 1
    xd = torch.from_numpy(xb.view(np.int16)).cuda()
    ro = torch.from_numpy(row_o).cuda()
    if op == "ct":
        want = ref.nv_quantize(xb, cols=True, want_y=False, given_outer=(row_o, col_o), **kw)
        co = None if col_o is None else torch.from_numpy(col_o).cuda()
        out = fq.fp4_cast_transpose(xd, g, row_outer=ro, col_outer=co)
        keys = ("row_codes", "row_scales", "col_codes", "col_scales")
    else:
        want = ref.nv_quantize(xb, want_y=False, given_outer=(row_o, col_o), **kw)
        out = fq.fp4_quantize(xd, g, outer=ro)
        out = {"row_codes": out["codes"], "row_scales": out["scales"]}
        keys = ("row_codes", "row_scales")
    for k in keys:
        _same(_host(out[k], np.uint8), want[k], k)
