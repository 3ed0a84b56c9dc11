"""Exact-rational model of the quantiser -- TEST INFRASTRUCTURE ONLY.

A second, independent statement of the same algorithm, used to pin the C
oracle (fp4_oracle.c) on small inputs.  Every value is a `fractions.Fraction`;
each binary32 operation is written as "compute the exact rational result, then
round it to the nearest binary32 (ties to even, subnormals kept)" by
`rn32`.  Grids are enumerated from their format definitions as rationals, and
every rounding onto a grid is an exact nearest-point search.  It shares no
code with fp4_oracle.c (which uses C float arithmetic and double-held grids).

Sources: "fp4-train" README (Method: block_absmax/6 scale, divide by the
decoded scale, E2M1 grid, stochastic rounding, error feedback); "NVFP4 /
AMD-FP4 outer-block (two-level) scaling" (Background, Technical design,
Implementation: outer scale amax/(scale_max*6) in FP32, normalise then inner
quantise); "MXFP4 weight QAT recipes" (Design, Correctness: 1x32 power-of-two
scales with floor 2^-126 and cap 2^125, block poisoning, signed zero).
SR draws are taken as an input array (the RNG is pinned separately).
"""
from fractions import Fraction as F

import numpy as np

E2M1 = [F(0), F(1, 2), F(1), F(3, 2), F(2), F(3), F(4), F(6)]


# --------------------------------------------------------------- binary32
def rn32(q: F) -> F:
    """Nearest binary32 value to the rational q (ties to even significand)."""
    if q == 0:
        return F(0)
    neg = q < 0
    a = -q if neg else q
    n, d = a.numerator, a.denominator
    e = n.bit_length() - d.bit_length()          # 2^e <= a < 2^(e+2) roughly
    if F(2) ** e > a:
        e -= 1
    while F(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                              # subnormal spacing below 2^-126
    ulp = F(2) ** (e - 23)
    m = a / ulp
    lo = m.numerator // m.denominator
    rem = m - lo
    if rem > F(1, 2) or (rem == F(1, 2) and lo % 2 == 1):
        lo += 1
    r = lo * ulp
    if r >= F(2) ** 128:
        raise OverflowError("binary32 overflow")
    return -r if neg else r


def f32_bits_to_frac(bits: int) -> F:
    bits &= 0xFFFFFFFF
    s = -1 if bits >> 31 else 1
    e = (bits >> 23) & 0xFF
    m = bits & 0x7FFFFF
    if e == 0xFF:
        raise ValueError("non-finite")
    if e == 0:
        return s * F(m) * F(2) ** (-149)
    return s * (1 + F(m, 1 << 23)) * F(2) ** (e - 127)


def bf16_to_frac(b: int) -> F:
    return f32_bits_to_frac((int(b) & 0xFFFF) << 16)


def bf16_sign(b: int) -> int:
    return (int(b) >> 15) & 1


def frac_to_bf16(q: F, neg_zero: bool = False) -> int:
    """RNE of a binary32-representable rational onto bf16 (8 significant bits)."""
    if q == 0:
        return 0x8000 if neg_zero else 0
    neg = q < 0
    a = -q if neg else q
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if F(2) ** e > a:
        e -= 1
    while F(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    ulp = F(2) ** (e - 7)
    m = a / ulp
    lo = m.numerator // m.denominator
    rem = m - lo
    if rem > F(1, 2) or (rem == F(1, 2) and lo % 2 == 1):
        lo += 1
    r = lo * ulp
    if r >= F(2) ** 128:
        return 0xFF80 if neg else 0x7F80
    # encode r as bf16 bits
    if r < F(2) ** -126:
        mant = int(r / F(2) ** -133)
        bits = mant
    else:
        ee = r.numerator.bit_length() - r.denominator.bit_length()
        if F(2) ** ee > r:
            ee -= 1
        mant = int((r / F(2) ** ee - 1) * 128)
        bits = ((ee + 127) << 7) | mant
    return bits | (0x8000 if neg else 0)


# --------------------------------------------------------------- grids
def scale_grid(fmt: str):
    """All finite non-negative values of the inner-scale format, index = code."""
    ebits, bias = (4, 7) if fmt == "e4m3" else (5, 15)
    top = 0x7E if fmt == "e4m3" else 0xFE
    vals = []
    for c in range(top + 1):
        e, m = c >> 3, c & 7
        if e == 0:
            vals.append(F(m, 8) * F(2) ** (1 - bias))
        else:
            vals.append(F(8 + m, 8) * F(2) ** (e - bias))
    return vals


_GRIDS = {}


def _grid(fmt):
    if fmt not in _GRIDS:
        _GRIDS[fmt] = scale_grid(fmt)
    return _GRIDS[fmt]


def nearest_even(value: F, grid) -> int:
    """Index of the grid point nearest to value; ties go to the even index;
    above the top point the top index (saturation)."""
    best, bestd = 0, abs(value - grid[0])
    for i in range(1, len(grid)):
        dd = abs(value - grid[i])
        if dd < bestd or (dd == bestd and i % 2 == 0):
            best, bestd = i, dd
    return best


def scale_encode(fmt: str, y: F) -> int:
    return nearest_even(y, _grid(fmt))


def scale_decode(fmt: str, c: int) -> F:
    return _grid(fmt)[c]


def e2m1_rne(t: F) -> int:
    return nearest_even(t, E2M1)


def e2m1_sr(t: F, u16: int) -> int:
    if t >= 6:
        return 7
    lo = max(i for i in range(8) if E2M1[i] <= t)
    if E2M1[lo] == t:
        return lo
    frac = (t - E2M1[lo]) / (E2M1[lo + 1] - E2M1[lo])
    return lo + 1 if F(u16, 65536) < frac else lo


# --------------------------------------------------------------- NVFP4 / AMD-FP4
def _bf16max():
    return bf16_to_frac(0x7F7F)


def _source_cell(b: int, f32: bool):
    """(kind, value, negative) of one source element given by its bf16 or
    binary32 bit pattern; kind is "nan", "inf" or "fin"."""
    ebits, mbits, sbit = (23, 0x7FFFFF, 31) if f32 else (7, 0x7F, 15)
    e = (b >> ebits) & 0xFF
    m = b & mbits
    neg = bool((b >> sbit) & 1)
    if e == 0xFF:
        return ("nan" if m else "inf"), None, neg
    return "fin", (f32_bits_to_frac(b) if f32 else bf16_to_frac(b)), neg


def _out_value(w: F, neg_zero: bool, f32: bool):
    """bf16 bits (RNE) or the float32 of a binary32-valued rational."""
    if not f32:
        return frac_to_bf16(w, neg_zero=neg_zero)
    if w == 0:
        return np.float32(-0.0 if neg_zero else 0.0)
    return np.float32(float(w))


def nv_quantize(x_bits, *, scale_fmt="e4m3", two_level="none", obs=0, outer_2d=False,
                stochastic=False, u16=None, residual=None, cols=False, inner_2d=False, y_f32=False):
    """Exact model of the NVFP4 / AMD-FP4 pipeline on a small [R, C] input.

    x_bits: uint16 bf16 bits, or uint32 binary32 bits (a binary32 source).
    residual: float32 array (read, not written; the new residual is returned).
    u16: uint16 [R, C] SR draws.  y_f32: dequantised outputs as float32 values
    instead of bf16 bits.  Returns a dict with the same buffers as the C oracle
    (numpy arrays)."""
    x_f32 = np.asarray(x_bits).dtype == np.uint32
    x_bits = np.asarray(x_bits, dtype=np.uint32 if x_f32 else np.uint16)
    R, C = x_bits.shape
    D = (F(448) if scale_fmt == "e4m3" else F(114688)) * 6
    D = rn32(D)
    # step 1: values (sanitised) and signs
    v = [[None] * C for _ in range(R)]
    vneg = [[False] * C for _ in range(R)]
    for i in range(R):
        for j in range(C):
            kind, xv, xn = _source_cell(int(x_bits[i, j]), x_f32)
            # sanitisation applies to the value being quantised: NaN -> +0,
            # +-inf -> +-largest bf16 (a non-finite x stays non-finite after
            # adding a finite residual, so it is sanitised directly)
            if kind == "nan":
                v[i][j], vneg[i][j] = F(0), False
                continue
            if kind == "inf":
                v[i][j], vneg[i][j] = (-_bf16max() if xn else _bf16max()), xn
                continue
            if residual is not None:
                zb = int(np.float32(residual[i, j]).view(np.uint32))
                z = f32_bits_to_frac(zb)
                try:
                    vv = rn32(xv + z)
                except OverflowError:
                    vv = _bf16max() if xv + z > 0 else -_bf16max()
                if vv == 0:
                    # IEEE: an exact zero sum is +0 unless both operands are -0
                    vneg[i][j] = xn and bool(zb >> 31) and xv == 0 and z == 0
                else:
                    vneg[i][j] = vv < 0
                v[i][j] = vv
            else:
                v[i][j] = xv
                vneg[i][j] = xn
    # step 2: outer scales
    def amax(cells):
        return max((abs(v[i][j]) for i, j in cells), default=F(0))

    row_outer = col_outer = None
    so_r = so_c = None
    if two_level == "tensorwise":
        s = rn32(amax([(i, j) for i in range(R) for j in range(C)]) / D)
        row_outer = np.array([float(s)], np.float32)
        so_r = lambda i, j: s  # noqa: E731
        so_c = so_r
    elif two_level == "outer" and outer_2d:
        TR, TC = R // obs, C // obs
        tiles = [[rn32(amax([(i, j) for i in range(ti * obs, (ti + 1) * obs)
                                  for j in range(tj * obs, (tj + 1) * obs)]) / D)
                  for tj in range(TC)] for ti in range(TR)]
        row_outer = np.array([[float(t) for t in r] for r in tiles], np.float32)
        so_r = lambda i, j: tiles[i // obs][j // obs]  # noqa: E731
        so_c = so_r
    elif two_level == "outer":
        rg = [[rn32(amax([(i, j) for j in range(g * obs, (g + 1) * obs)]) / D) for g in range(C // obs)]
              for i in range(R)]
        row_outer = np.array([[float(t) for t in r] for r in rg], np.float32)
        so_r = lambda i, j: rg[i][j // obs]  # noqa: E731
        if cols:
            cg = [[rn32(amax([(i, j) for i in range(g * obs, (g + 1) * obs)]) / D) for g in range(R // obs)]
                  for j in range(C)]
            col_outer = np.array([[float(t) for t in r] for r in cg], np.float32)
            so_c = lambda i, j: cg[j][i // obs]  # noqa: E731

    def normalised(i, j, so):
        if so is None:
            return v[i][j], vneg[i][j]
        s = so(i, j)
        if s == 0:
            return F(0), vneg[i][j]
        q = rn32(v[i][j] / s)
        return q, (q < 0) if q != 0 else vneg[i][j]

    def tile_max(i0, j0, so):
        """largest |normalised value| of the 16 x 16 tile with corner (i0, j0) (2D inner scaling)"""
        return max(abs(normalised(i, j, so)[0]) for i in range(i0, i0 + 16) for j in range(j0, j0 + 16))

    def quant_block(vals, b=None):
        """vals: list of (value, neg, u16) for one 16-block -> (scale code, d, [(code, p)]);
        b: the block amax, when it comes from the enclosing 16 x 16 tile"""
        if b is None:
            b = max(abs(a) for a, _, _ in vals)
        y = rn32(b / 6)
        cs = scale_encode(scale_fmt, y)
        d = scale_decode(scale_fmt, cs)
        res = []
        for a, neg, u in vals:
            t = F(0) if d == 0 else rn32(abs(a) / d)
            m = e2m1_sr(t, u) if stochastic else e2m1_rne(t)
            res.append(((8 if neg else 0) | m, E2M1[m] * d))
        return cs, d, res

    def draws(i, j):
        return int(u16[i, j]) if stochastic else 0

    out = {}
    row_codes = np.zeros((R, C // 2), np.uint8)
    row_scales = np.zeros((R, C // 16), np.uint8)
    row_y = np.zeros((R, C), np.float32 if y_f32 else np.uint16)
    new_res = np.zeros((R, C), np.float32) if residual is not None else None
    for i in range(R):
        for j0 in range(0, C, 16):
            vals = []
            for j in range(j0, j0 + 16):
                a, neg = normalised(i, j, so_r)
                vals.append((a, neg, draws(i, j)))
            cs, d, res = quant_block(vals, tile_max(i - i % 16, j0, so_r) if inner_2d else None)
            row_scales[i, j0 // 16] = cs
            for k, (code, p) in enumerate(res):
                j = j0 + k
                row_codes[i, j // 2] |= (code << 4) if (j & 1) else code
                w = p if so_r is None else rn32(p * so_r(i, j))
                neg = bool(code & 8)
                wv = -w if neg else w
                row_y[i, j] = _out_value(wv, neg and w == 0, y_f32)
                if new_res is not None:
                    r = rn32(v[i][j] - wv)
                    if r == 0:
                        # exact-zero difference: +0 (IEEE), unless v is -0 and w is +0
                        rneg = vneg[i][j] and v[i][j] == 0 and not (neg and w == 0) and w == 0
                        new_res[i, j] = -0.0 if rneg else 0.0
                    else:
                        new_res[i, j] = np.float32(float(r))
    out.update(row_codes=row_codes, row_scales=row_scales, row_y=row_y)
    if row_outer is not None:
        out["row_outer"] = row_outer
    if new_res is not None:
        out["residual"] = new_res
    if cols:
        col_codes = np.zeros((C, R // 2), np.uint8)
        col_scales = np.zeros((C, R // 16), np.uint8)
        col_y = np.zeros((C, R), np.float32 if y_f32 else np.uint16)
        for j in range(C):
            for i0 in range(0, R, 16):
                vals = []
                for i in range(i0, i0 + 16):
                    a, neg = normalised(i, j, so_c)
                    vals.append((a, neg, draws(i, j)))
                cs, d, res = quant_block(vals, tile_max(i0, j - j % 16, so_c) if inner_2d else None)
                col_scales[j, i0 // 16] = cs
                for k, (code, p) in enumerate(res):
                    i = i0 + k
                    col_codes[j, i // 2] |= (code << 4) if (i & 1) else code
                    w = p if so_c is None else rn32(p * so_c(i, j))
                    neg = bool(code & 8)
                    col_y[j, i] = _out_value(-w if neg else w, neg and w == 0, y_f32)
        out.update(col_codes=col_codes, col_scales=col_scales, col_y=col_y)
        if col_outer is not None:
            out["col_outer"] = col_outer
    return out


# --------------------------------------------------------------- MXFP4
def mx_qdq(x_bits, y_f32=False):
    """Exact model of the MXFP4 1x32 fake-quant: (codes, scales, y).  x_bits:
    uint16 bf16 bits or uint32 binary32 bits; y as bf16 bits, or float32
    values with y_f32."""
    x_f32 = np.asarray(x_bits).dtype == np.uint32
    x_bits = np.asarray(x_bits, dtype=np.uint32 if x_f32 else np.uint16)
    R, C = x_bits.shape
    codes = np.zeros((R, C // 2), np.uint8)
    scales = np.zeros((R, C // 32), np.uint8)
    y = np.zeros((R, C), np.float32 if y_f32 else np.uint16)
    for i in range(R):
        for j0 in range(0, C, 32):
            cells = [_source_cell(int(b), x_f32) for b in x_bits[i, j0:j0 + 32]]
            if any(kind != "fin" for kind, _, _ in cells):
                scales[i, j0 // 32] = 0xFF
                y[i, j0:j0 + 32] = np.float32("nan") if y_f32 else 0x7FC0
                continue
            A = max(abs(val) for _, val, _ in cells)
            if A == 0:
                k = -126
            else:
                # smallest k with A <= 6 * 2^k, searched from far below
                k = -300
                while 6 * F(2) ** k < A:
                    k += 1
                k = min(max(k, -126), 125)
            scales[i, j0 // 32] = k + 127
            for kk, (_, val, neg) in enumerate(cells):
                j = j0 + kk
                t = abs(val) / F(2) ** k
                m = e2m1_rne(t)
                code = (8 if neg else 0) | m
                codes[i, j // 2] |= (code << 4) if (j & 1) else code
                w = E2M1[m] * F(2) ** k
                y[i, j] = _out_value(-w if neg else w, neg and w == 0, y_f32)
    return codes, scales, y
