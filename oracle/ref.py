"""ctypes binding of the C oracle (fp4_oracle.c) -- TEST INFRASTRUCTURE ONLY.

Arrays are numpy; bf16 tensors travel as uint16 bit patterns.  Every function
here only marshals arguments; the arithmetic is in fp4_oracle.c.
"""
import ctypes as ct
import os

import numpy as np

from . import build as _build

_lib = None

SCALE_FMT = {"e4m3": 1, "ue5m3": 2}
TWO_LEVEL = {"none": 0, "tensorwise": 1, "outer": 2}


class _NvParams(ct.Structure):
    _fields_ = [("scale_fmt", ct.c_int32), ("two_level", ct.c_int32), ("obs", ct.c_int32),
                ("outer_2d", ct.c_int32), ("stochastic", ct.c_int32), ("use_given_outer", ct.c_int32),
                ("inner_2d", ct.c_int32),
                ("seed", ct.c_uint64), ("step", ct.c_uint64), ("index_base", ct.c_uint64)]


def lib():
    global _lib
    if _lib is None:
        path = _build.LIB
        if os.environ.get("FP4Q_SANITIZE") == "1":
            # the UBSan build (sanitizer runs of the CPU suite)
            path = _build.LIB_UBSAN
            if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
                _build.build_ubsan()
        elif not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
        L = ct.CDLL(path)
        P = ct.c_void_p
        L.orc_bf16_to_f32.restype = ct.c_float
        L.orc_bf16_to_f32.argtypes = [ct.c_uint16]
        L.orc_f32_to_bf16.restype = ct.c_uint16
        L.orc_f32_to_bf16.argtypes = [ct.c_float]
        L.orc_e2m1_value.restype = ct.c_double
        L.orc_e2m1_value.argtypes = [ct.c_int]
        L.orc_e2m1_rne.restype = ct.c_int
        L.orc_e2m1_rne.argtypes = [ct.c_double]
        L.orc_e2m1_sr.restype = ct.c_int
        L.orc_e2m1_sr.argtypes = [ct.c_double, ct.c_uint32]
        L.orc_scale_decode.restype = ct.c_double
        L.orc_scale_decode.argtypes = [ct.c_int, ct.c_int]
        L.orc_scale_encode.restype = ct.c_int
        L.orc_scale_encode.argtypes = [ct.c_int, ct.c_float]
        L.orc_ue8m0_decode.restype = ct.c_double
        L.orc_ue8m0_decode.argtypes = [ct.c_int]
        L.orc_philox4x32_10.restype = None
        L.orc_philox4x32_10.argtypes = [P, P, P]
        L.orc_sr_u16.restype = ct.c_uint32
        L.orc_sr_u16.argtypes = [ct.c_uint64, ct.c_uint64, ct.c_uint64]
        L.orc_max_threads.restype = ct.c_int
        L.orc_max_threads.argtypes = []
        L.orc_set_threads.restype = None
        L.orc_set_threads.argtypes = [ct.c_int]
        for name in ("orc_f32_to_bf16_array", "orc_e2m1_rne_array"):
            getattr(L, name).restype = None
            getattr(L, name).argtypes = [P, ct.c_int64, P]
        L.orc_scale_encode_array.restype = None
        L.orc_scale_encode_array.argtypes = [ct.c_int, P, ct.c_int64, P]
        L.orc_sr_u16_array.restype = None
        L.orc_sr_u16_array.argtypes = [ct.c_uint64, ct.c_uint64, ct.c_uint64, ct.c_int64, P]
        L.orc_div_array.restype = None
        L.orc_div_array.argtypes = [P, P, ct.c_int64, P]
        L.orc_nv_quantize.restype = ct.c_int
        L.orc_nv_quantize.argtypes = [ct.POINTER(_NvParams), P, ct.c_int64, ct.c_int64, P,
                                      P, P, P, P, P, P, P, P]
        L.orc_nv_quantize_ex.restype = ct.c_int
        L.orc_nv_quantize_ex.argtypes = [ct.POINTER(_NvParams), P, ct.c_int, ct.c_int64, ct.c_int64, P,
                                         P, P, P, P, P, P, P, P, ct.c_int]
        L.orc_nv_dequantize_ex.restype = ct.c_int
        L.orc_nv_dequantize_ex.argtypes = [ct.c_int, ct.c_int, ct.c_int64, P, P, P,
                                           ct.c_int64, ct.c_int64, P, ct.c_int]
        L.orc_mx_qdq_ex.restype = ct.c_int
        L.orc_mx_qdq_ex.argtypes = [P, ct.c_int, ct.c_int64, ct.c_int64, P, P, P, ct.c_int]
        L.orc_mx_dequantize_ex.restype = ct.c_int
        L.orc_mx_dequantize_ex.argtypes = [P, P, ct.c_int64, ct.c_int64, P, ct.c_int]
        L.orc_mx_mm.restype = ct.c_int
        L.orc_mx_mm.argtypes = [P, P, P, P, ct.c_int64, ct.c_int64, ct.c_int64, P, P]
        L.orc_nv_quantize_grouped.restype = ct.c_int
        L.orc_nv_quantize_grouped.argtypes = [ct.POINTER(_NvParams), ct.c_int32, P, ct.c_int64,
                                              P, P, P, P, P, P, P, P]
        L.orc_nv_dequantize.restype = ct.c_int
        L.orc_nv_dequantize.argtypes = [ct.c_int, ct.c_int, ct.c_int64, P, P, P,
                                        ct.c_int64, ct.c_int64, P]
        L.orc_mx_qdq.restype = ct.c_int
        L.orc_mx_qdq.argtypes = [P, ct.c_int64, ct.c_int64, P, P, P]
        L.orc_mx_project_encode.restype = ct.c_int
        L.orc_mx_project_encode.argtypes = [P, ct.c_int64, ct.c_int64, P, P, P, P, P, P, P, P]
        L.orc_e4m3_payload.restype = ct.c_uint8
        L.orc_e4m3_payload.argtypes = [ct.c_double]
        L.orc_mx_dequantize.restype = ct.c_int
        L.orc_mx_dequantize.argtypes = [P, P, ct.c_int64, ct.c_int64, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ct.c_void_p)


def threads() -> int:
    return lib().orc_max_threads()


def set_threads(n: int) -> None:
    """OpenMP thread count of the oracle's parallel loops (timing only)."""
    lib().orc_set_threads(int(n))


# ---------------------------------------------------------------- primitives
def bf16_to_f32(bits):
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(f):
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, np.uint16)
    lib().orc_f32_to_bf16_array(_p(f), f.size, _p(out))
    return out


def e2m1_value(m: int) -> float:
    return lib().orc_e2m1_value(int(m))


def e2m1_rne(a: float) -> int:
    return lib().orc_e2m1_rne(float(a))


def e2m1_rne_array(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, np.uint8)
    lib().orc_e2m1_rne_array(_p(a), a.size, _p(out))
    return out


def e2m1_sr(a: float, u16: int) -> int:
    return lib().orc_e2m1_sr(float(a), int(u16))


def scale_decode(fmt: str, code: int) -> float:
    return lib().orc_scale_decode(SCALE_FMT[fmt], int(code))


def scale_encode(fmt: str, y: float) -> int:
    return lib().orc_scale_encode(SCALE_FMT[fmt], float(y))


def scale_encode_array(fmt: str, y):
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, np.uint8)
    lib().orc_scale_encode_array(SCALE_FMT[fmt], _p(y), y.size, _p(out))
    return out


def ue8m0_decode(code: int) -> float:
    return lib().orc_ue8m0_decode(int(code))


def philox4x32_10(ctr, key):
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.empty(4, np.uint32)
    lib().orc_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def sr_u16(seed: int, step: int, idx: int) -> int:
    return lib().orc_sr_u16(seed, step, idx)


def sr_u16_array(seed: int, step: int, idx0: int, n: int):
    out = np.empty(n, np.uint16)
    lib().orc_sr_u16_array(seed, step, idx0, n, _p(out))
    return out


def div_f32(a, b):
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    out = np.empty(a.shape, np.float32)
    lib().orc_div_array(_p(a), _p(b), a.size, _p(out))
    return out


# ---------------------------------------------------------------- algorithms
def _params(scale_fmt, two_level, obs, outer_2d, stochastic, seed, step, index_base, given, inner_2d=False):
    return _NvParams(SCALE_FMT[scale_fmt], TWO_LEVEL[two_level], int(obs), int(bool(outer_2d)),
                     int(bool(stochastic)), int(bool(given)), int(bool(inner_2d)), int(seed), int(step),
                     int(index_base))


def outer_shapes(two_level, obs, outer_2d, R, C):
    """(row_outer shape, col_outer shape or None) for an [R, C] source."""
    if two_level == "none":
        return None, None
    if two_level == "tensorwise":
        return (1,), None
    if outer_2d:
        return (R // obs, C // obs), None
    return (R, C // obs), (C, R // obs)


def _source(x):
    """(contiguous array, 1 if binary32) of a source given as uint16 bf16 bits
    or as float32 values."""
    if np.asarray(x).dtype == np.float32:
        return np.ascontiguousarray(x, dtype=np.float32), 1
    return np.ascontiguousarray(x, dtype=np.uint16), 0


_Y_DT = {"bf16": np.uint16, "fp32": np.float32}


def nv_quantize(x, *, scale_fmt="e4m3", two_level="none", obs=0, outer_2d=False,
                stochastic=False, seed=0, step=0, index_base=0, residual=None,
                given_outer=None, cols=False, want_y=True, inner_2d=False, y_dtype="bf16"):
    """Oracle NVFP4 / AMD-FP4 quantisation of x ([R, C]: uint16 bf16 bits, or
    float32 values for a binary32 source).

    y_dtype: "bf16" (row_y / col_y as uint16 bits) or "fp32" (float32 values).

    residual: float32 [R, C] updated in place (error feedback) or None.
    given_outer: (row_outer, col_outer) supplied by the caller instead of computed.
    inner_2d: 16 x 16 inner tiles share one scale (replicated in each of their 16
    rows of row_scales; the columnwise buffers are the transposes).
    Returns a dict of numpy arrays.
    """
    x, x_f32 = _source(x)
    ydt = _Y_DT[y_dtype]
    R, C = x.shape
    out = {"row_codes": np.zeros((R, C // 2), np.uint8), "row_scales": np.zeros((R, C // 16), np.uint8)}
    rs, cs = outer_shapes(two_level, obs, outer_2d, R, C)
    if given_outer is not None:
        out["row_outer"] = np.ascontiguousarray(given_outer[0], dtype=np.float32).copy()
        if cs is not None and cols:
            out["col_outer"] = np.ascontiguousarray(given_outer[1], dtype=np.float32).copy()
    else:
        if rs is not None:
            out["row_outer"] = np.zeros(rs, np.float32)
        if cs is not None and cols:
            out["col_outer"] = np.zeros(cs, np.float32)
    if want_y:
        out["row_y"] = np.zeros((R, C), ydt)
    if cols:
        out["col_codes"] = np.zeros((C, R // 2), np.uint8)
        out["col_scales"] = np.zeros((C, R // 16), np.uint8)
        if want_y:
            out["col_y"] = np.zeros((C, R), ydt)
    if residual is not None:
        assert residual.dtype == np.float32 and residual.flags.c_contiguous and residual.shape == (R, C)
    prm = _params(scale_fmt, two_level, obs, outer_2d, stochastic, seed, step, index_base, given_outer is not None,
                  inner_2d)
    rc = lib().orc_nv_quantize_ex(ct.byref(prm), _p(x), x_f32, R, C, _p(residual),
                                  _p(out["row_codes"]), _p(out["row_scales"]), _p(out.get("row_outer")),
                                  _p(out.get("row_y")), _p(out.get("col_codes")), _p(out.get("col_scales")),
                                  _p(out.get("col_outer")), _p(out.get("col_y")), int(y_dtype == "fp32"))
    if rc != 0:
        raise ValueError("oracle rejected the configuration (%d)" % rc)
    return out


def nv_quantize_grouped(x, rows, *, scale_fmt="e4m3", two_level="outer", obs=64, outer_2d=True,
                        stochastic=False, seed=0, step=0, index_base=0, residual=None, inner_2d=False):
    """Per-group (expert) quantisation of stacked x [sum(rows), C], both directions."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    total, C = x.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    assert rows.sum() == total
    n_outer_r = n_outer_c = 0
    for R in rows:
        rs, cs = outer_shapes(two_level, obs, outer_2d, int(R), C)
        n_outer_r += int(np.prod(rs)) if rs else 0
        n_outer_c += int(np.prod(cs)) if cs else 0
    out = {"row_codes": np.zeros((total, C // 2), np.uint8), "row_scales": np.zeros((total, C // 16), np.uint8),
           "col_codes": np.zeros((total * C // 2,), np.uint8), "col_scales": np.zeros((total * C // 16,), np.uint8),
           "row_outer": np.zeros(max(n_outer_r, 1), np.float32), "col_outer": np.zeros(max(n_outer_c, 1), np.float32)}
    prm = _params(scale_fmt, two_level, obs, outer_2d, stochastic, seed, step, index_base, False, inner_2d)
    rc = lib().orc_nv_quantize_grouped(ct.byref(prm), len(rows), _p(rows), C, _p(x), _p(residual),
                                       _p(out["row_codes"]), _p(out["row_scales"]), _p(out["row_outer"]),
                                       _p(out["col_codes"]), _p(out["col_scales"]), _p(out["col_outer"]))
    if rc != 0:
        raise ValueError("oracle rejected the configuration (%d)" % rc)
    out["row_outer"] = out["row_outer"][:n_outer_r]
    out["col_outer"] = out["col_outer"][:n_outer_c]
    return out


OUTER_KIND = {"none": 0, "tensorwise": 1, "1d": 2, "2d": 3, "2d_t": 4}


def nv_dequantize(codes, scales, outer, R, C, *, scale_fmt="e4m3", outer_kind="none", obs=0, y_dtype="bf16"):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    outer = None if outer is None else np.ascontiguousarray(outer, dtype=np.float32)
    y = np.zeros((R, C), _Y_DT[y_dtype])
    rc = lib().orc_nv_dequantize_ex(SCALE_FMT[scale_fmt], OUTER_KIND[outer_kind], int(obs),
                                    _p(codes), _p(scales), _p(outer), R, C, _p(y), int(y_dtype == "fp32"))
    if rc != 0:
        raise ValueError("oracle rejected the configuration (%d)" % rc)
    return y


def mx_qdq(x, y_dtype="bf16"):
    """MXFP4 fake-quant of x (uint16 bf16 bits, or float32 values): returns
    (codes [R, C/2], scales [R, C/32], y [R, C] as bf16 bits or float32)."""
    x, x_f32 = _source(x)
    R, C = x.shape
    codes = np.zeros((R, C // 2), np.uint8)
    scales = np.zeros((R, C // 32), np.uint8)
    y = np.zeros((R, C), _Y_DT[y_dtype])
    rc = lib().orc_mx_qdq_ex(_p(x), x_f32, R, C, _p(codes), _p(scales), _p(y), int(y_dtype == "fp32"))
    if rc != 0:
        raise ValueError("oracle rejected the shape (%d)" % rc)
    return codes, scales, y


def e4m3_payload(v):
    """E4M3 payload byte of one value (RNE, subnormals, sign kept, NaN -> 0xFF)."""
    return int(lib().orc_e4m3_payload(float(v)))


def mx_project_encode(x, *, y=True, mx8_row=True, mx8_col=True, blk=True):
    """MXFP4 projection of x (bf16 bits [R, C]) and its FP8 re-encodings.

    Returns a dict with any of: y (bf16 bits [R, C]); mx8_row (E4M3 [R, C]) and
    mx8_row_scales (UE8M0 [R, C/32]); mx8_col (E4M3 [C, R]) and mx8_col_scales
    (UE8M0 [C, R/32]); blk (E4M3 [R, C]), blk_t (E4M3 [C, R]) and blk_scales
    (FP32 [R/128, C/128]).
    """
    x = np.ascontiguousarray(x, dtype=np.uint16)
    R, C = x.shape
    out = {}
    if y:
        out["y"] = np.zeros((R, C), np.uint16)
    if mx8_row:
        out["mx8_row"] = np.zeros((R, C), np.uint8)
        out["mx8_row_scales"] = np.zeros((R, C // 32), np.uint8)
    if mx8_col:
        out["mx8_col"] = np.zeros((C, R), np.uint8)
        out["mx8_col_scales"] = np.zeros((C, R // 32), np.uint8)
    if blk:
        out["blk"] = np.zeros((R, C), np.uint8)
        out["blk_t"] = np.zeros((C, R), np.uint8)
        out["blk_scales"] = np.zeros((R // 128, C // 128), np.float32)
    g = out.get
    rc = lib().orc_mx_project_encode(_p(x), R, C, _p(g("y")), _p(g("mx8_row")), _p(g("mx8_row_scales")),
                                     _p(g("mx8_col")), _p(g("mx8_col_scales")), _p(g("blk")), _p(g("blk_t")),
                                     _p(g("blk_scales")))
    if rc != 0:
        raise ValueError("oracle rejected the shape (%d)" % rc)
    return out


def mx_dequantize(codes, scales, R, C, y_dtype="bf16"):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    y = np.zeros((R, C), _Y_DT[y_dtype])
    rc = lib().orc_mx_dequantize_ex(_p(codes), _p(scales), R, C, _p(y), int(y_dtype == "fp32"))
    if rc != 0:
        raise ValueError("oracle rejected the shape (%d)" % rc)
    return y


def mx_mm(a_codes, a_scales, b_codes, b_scales, M, N, K):
    """C = A . B^T of MXFP4 operands (rowwise codes [*, K/2], UE8M0 scales
    [*, K/32]) in binary64: returns (c, s), s the sum of |products| per entry."""
    a_codes = np.ascontiguousarray(a_codes, dtype=np.uint8)
    a_scales = np.ascontiguousarray(a_scales, dtype=np.uint8)
    b_codes = np.ascontiguousarray(b_codes, dtype=np.uint8)
    b_scales = np.ascontiguousarray(b_scales, dtype=np.uint8)
    c = np.zeros((M, N), np.float64)
    s = np.zeros((M, N), np.float64)
    rc = lib().orc_mx_mm(_p(a_codes), _p(a_scales), _p(b_codes), _p(b_scales), M, N, K, _p(c), _p(s))
    if rc != 0:
        raise ValueError("oracle rejected the shape (%d)" % rc)
    return c, s


def mx_scales_tiled(scales, rows, K):
    """GEMM-ready scale layout (a byte layout convention; parity unpinned):
    entry [t][kt][r][j] = scales[256 t + r][8 kt + j], 0 outside the input;
    returned flat (uint8)."""
    scales = np.asarray(scales, dtype=np.uint8).reshape(rows, K // 32)
    T, KT = -(-rows // 256), -(-K // 256)
    out = np.zeros((T, KT, 256, 8), np.uint8)
    for t in range(T):
        for kt in range(KT):
            for r in range(256):
                row = 256 * t + r
                if row >= rows:
                    break
                for j in range(8):
                    col = 8 * kt + j
                    if col < K // 32:
                        out[t, kt, r, j] = scales[row, col]
    return out.ravel()
