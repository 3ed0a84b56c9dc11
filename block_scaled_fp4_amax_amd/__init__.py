"""block_scaled_fp4_amax_amd -- Python binding of libfp4q.so, the gfx950
block-scaled FP4 quantisation library.

The functions carry the C-ABI names (fp4_quantize, fp4_dequantize, fp4_qdq,
fp4_cast_transpose, fp4_cast_transpose_grouped and the fp4q_* helpers).  They
only marshal arguments: torch supplies device memory and the current HIP
stream, every step of the computation runs in the library's HIP kernels.  If
the library is not built, importing the binding raises; there is no fallback.

Layouts, numerics and error rules are those documented in include/fp4q.h.
"""
import ctypes as ct
import os

__all__ = [
    "Fp4Error", "Cfg", "Sizes", "make_cfg", "lib", "fp4q_abi_version", "fp4q_status_str", "fp4q_buffer_sizes",
    "fp4q_workspace_bytes", "fp4q_cast_transpose_workspace_bytes", "fp4_quantize", "fp4_dequantize", "fp4_qdq", "fp4_cast_transpose",
    "fp4_cast_transpose_grouped", "fp4_mx_project_fp8", "fp4_mm", "fp4_mx_scales_tiled",
    "fp4q_mx_scales_tiled_bytes", "fp4_qdq_noalloc", "ErrorFeedback", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "libfp4q_ubsan.so" if os.environ.get("FP4Q_SANITIZE") == "1" else "libfp4q.so")

OK, ERR_NULL, ERR_DTYPE, ERR_SHAPE, ERR_MODE, ERR_UNSUPPORTED, ERR_ALIGN, ERR_WORKSPACE, ERR_HIP, ERR_ABI = range(10)
ABI_VERSION = 2

FORMATS = {"nvfp4": 0, "amdfp4": 1, "mxfp4": 2}
SCALE_FORMATS = {None: 0, "default": 0, "e4m3": 1, "ue5m3": 2, "ue8m0": 3}
TWO_LEVEL = {"none": 0, "tensorwise": 1, "outer_block": 2}
ROUNDING = {"rne": 0, "stochastic": 1}
DTYPES = {"bf16": 0, "fp16": 1, "fp32": 2}


class Fp4Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, fp4q_status_str(status), status))


class Cfg(ct.Structure):
    _fields_ = [("abi_version", ct.c_uint32), ("format", ct.c_int32), ("scale_format", ct.c_int32),
                ("two_level", ct.c_int32), ("outer_block_size", ct.c_int32), ("outer_2d", ct.c_int32),
                ("rounding", ct.c_int32), ("outer_mode", ct.c_int32), ("input_dtype", ct.c_int32),
                ("inner_2d", ct.c_int32), ("output_dtype", ct.c_int32), ("seed", ct.c_uint64),
                ("step", ct.c_uint64), ("index_base", ct.c_uint64)]


class Sizes(ct.Structure):
    _fields_ = [(n, ct.c_size_t) for n in ("row_codes", "row_scales", "row_outer", "col_codes", "col_scales",
                                           "col_outer", "y", "residual", "workspace")]


def make_cfg(format="nvfp4", scale_format=None, two_level="none", outer_block_size=0, outer_2d=False,
             rounding="rne", outer_mode=0, seed=0, step=0, index_base=0, input_dtype="bf16", inner_2d=False,
             output_dtype="bf16"):
    """Build an fp4q_cfg (string names or the raw integers of include/fp4q.h).

    inner_2d: one inner scale per 16 x 16 tile instead of per 1 x 16 block.
    input_dtype / output_dtype: "bf16" or "fp32" (the entry points below set
    them from the tensors they are given)."""
    def pick(table, v):
        return v if isinstance(v, int) and not isinstance(v, bool) else table[v]
    return Cfg(ABI_VERSION, pick(FORMATS, format), pick(SCALE_FORMATS, scale_format), pick(TWO_LEVEL, two_level),
               int(outer_block_size), int(bool(outer_2d)), pick(ROUNDING, rounding), int(outer_mode),
               pick(DTYPES, input_dtype), int(inner_2d), pick(DTYPES, output_dtype), int(seed), int(step),
               int(index_base))


def _with_dtypes(cfg, input_dtype=None, output_dtype=None):
    """A copy of cfg with its dtype fields set from the tensors of a call."""
    c = Cfg.from_buffer_copy(cfg)
    if input_dtype is not None:
        c.input_dtype = DTYPES[input_dtype]
    if output_dtype is not None:
        c.output_dtype = DTYPES[output_dtype]
    return c


_lib = None


def lib():
    """The loaded libfp4q.so (ctypes), with argument types declared."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libfp4q.so is not built (run __graft_entry__.build() or "
                              "python block_scaled_fp4_amax_amd/build.py)")
        L = ct.CDLL(LIB_PATH)
        P, I64, SZ = ct.c_void_p, ct.c_int64, ct.c_size_t
        C = ct.POINTER(Cfg)
        L.fp4q_abi_version.restype = ct.c_uint32
        L.fp4q_abi_version.argtypes = []
        L.fp4q_status_str.restype = ct.c_char_p
        L.fp4q_status_str.argtypes = [ct.c_int]
        L.fp4q_buffer_sizes.restype = ct.c_int
        L.fp4q_buffer_sizes.argtypes = [C, I64, I64, ct.POINTER(Sizes)]
        L.fp4q_workspace_bytes.restype = SZ
        L.fp4q_workspace_bytes.argtypes = [C, I64, I64]
        L.fp4q_cast_transpose_workspace_bytes.restype = SZ
        L.fp4q_cast_transpose_workspace_bytes.argtypes = [C, ct.c_int32, P, I64, ct.c_int32]
        L.fp4_quantize.restype = ct.c_int
        L.fp4_quantize.argtypes = [C, P, I64, I64, I64, P, P, P, P, P, SZ, P]
        L.fp4_dequantize.restype = ct.c_int
        L.fp4_dequantize.argtypes = [C, P, P, P, I64, I64, ct.c_int32, P, P]
        L.fp4_qdq.restype = ct.c_int
        L.fp4_qdq.argtypes = [C, P, I64, I64, I64, P, P, P, P, P, P, SZ, P]
        L.fp4_qdq_noalloc.restype = ct.c_int
        L.fp4_qdq_noalloc.argtypes = [C, P, I64, I64, I64, P, P, P, P, P, P]
        L.fp4_cast_transpose.restype = ct.c_int
        L.fp4_cast_transpose.argtypes = [C, P, I64, I64, I64, P, P, P, P, P, P, P, P, SZ, P]
        L.fp4_cast_transpose_grouped.restype = ct.c_int
        L.fp4_cast_transpose_grouped.argtypes = [C, ct.c_int32, P, I64, P, I64, P, P, P, P, P, P, P, P, SZ, P]
        L.fp4_mm.restype = ct.c_int
        L.fp4_mm.argtypes = [C, P, P, P, P, I64, I64, I64, ct.c_int32, P, I64, P]
        L.fp4q_mx_scales_tiled_bytes.restype = SZ
        L.fp4q_mx_scales_tiled_bytes.argtypes = [I64, I64]
        L.fp4_mx_scales_tiled.restype = ct.c_int
        L.fp4_mx_scales_tiled.argtypes = [P, I64, I64, P, P]
        L.fp4_mx_project_fp8.restype = ct.c_int
        L.fp4_mx_project_fp8.argtypes = [C, P, I64, I64, I64, P, P, P, P, P, P, P, P, P]
        if L.fp4q_abi_version() != ABI_VERSION:
            raise ImportError("libfp4q.so ABI %d, binding expects %d" % (L.fp4q_abi_version(), ABI_VERSION))
        _lib = L
    return _lib


def fp4q_abi_version():
    return lib().fp4q_abi_version()


def fp4q_status_str(status):
    return lib().fp4q_status_str(int(status)).decode()


def fp4q_buffer_sizes(cfg, rows, cols):
    s = Sizes()
    st = lib().fp4q_buffer_sizes(ct.byref(cfg), int(rows), int(cols), ct.byref(s))
    if st:
        raise Fp4Error(st, "fp4q_buffer_sizes")
    return {n: getattr(s, n) for n, _ in Sizes._fields_}


def fp4q_workspace_bytes(cfg, rows, cols):
    return lib().fp4q_workspace_bytes(ct.byref(cfg), int(rows), int(cols))


def fp4q_cast_transpose_workspace_bytes(cfg, rows_per_group, cols, with_residual=False):
    """Workspace that lets the cast-transpose stage its outputs (see
    include/fp4q.h); rows_per_group is a list of row counts (one entry for a
    single tensor)."""
    rows = [int(r) for r in rows_per_group]
    arr = (ct.c_int64 * max(len(rows), 1))(*rows)
    return lib().fp4q_cast_transpose_workspace_bytes(ct.byref(cfg), len(rows), arr, int(cols), int(bool(with_residual)))


def _ct_workspace(cfg, rows, cols, residual, device, workspace, staged):
    """(workspace, bytes) for a cast-transpose call: the caller's, or one
    sized for staged outputs (staged=True) or for the tensorwise scratch only."""
    if workspace is not None:
        return workspace, workspace.numel() * workspace.element_size()
    nb = fp4q_cast_transpose_workspace_bytes(cfg, rows, cols, residual is not None) if staged else \
        fp4q_workspace_bytes(cfg, sum(rows), cols)
    if nb == 0:
        return None, 0
    return _empty(nb, _torch().uint8, device), nb


# ------------------------------------------------------------------ marshalling helpers
def _torch():
    import torch
    return torch


def _ptr(t):
    """Device address of a tensor (None for None).  Host tensors are refused:
    every pointer the library takes is a device pointer."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("fp4q takes device tensors; got one on %s" % t.device)
    return ct.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    if stream is None:
        return ct.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ct.c_void_p(stream)
    return ct.c_void_p(stream.cuda_stream)


def _check(st, where):
    if st:
        raise Fp4Error(st, where)


def _src(x, allow_f32=False):
    """(tensor, rows, cols, ld) for a 2-D bf16 (or 16-bit integer) source, or
    a float32 one where the entry point takes FP32."""
    torch = _torch()
    if x.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    ok = (torch.bfloat16, torch.int16, torch.uint16) + ((torch.float32,) if allow_f32 else ())
    if x.dtype not in ok:
        raise Fp4Error(ERR_DTYPE, "source dtype %s" % x.dtype)
    if x.shape[1] > 1 and x.stride(1) != 1:
        raise ValueError("source rows must be contiguous (stride(1) == 1)")
    ld = x.stride(0) if x.shape[0] > 1 else x.shape[1]
    return x, x.shape[0], x.shape[1], ld


def _need(t, nbytes, what):
    """A caller-supplied buffer must be contiguous and hold at least nbytes
    (the library trusts its buffer sizes, so this is checked before any call)."""
    if t is None:
        return
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % what)
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError("%s holds %d bytes, needs %d" % (what, have, nbytes))


def _need_residual(residual, R, C):
    if residual is None:
        return
    if residual.dtype != _torch().float32 or tuple(residual.shape) != (R, C):
        raise ValueError("residual must be a float32 [%d, %d] tensor" % (R, C))
    _need(residual, R * C * 4, "residual")


def _dtype_name(t):
    return "fp32" if t.dtype == _torch().float32 else "bf16"


def _empty(n, dtype, device):
    torch = _torch()
    return torch.empty(int(n), dtype=dtype, device=device)


def _inner(cfg):
    return 32 if cfg.format == FORMATS["mxfp4"] else 16


def _workspace(cfg, rows, cols, device, workspace):
    nb = fp4q_workspace_bytes(cfg, rows, cols)
    if nb == 0:
        return None, 0
    if workspace is None:
        workspace = _empty(nb, _torch().uint8, device)
    return workspace, workspace.numel() * workspace.element_size()


# ------------------------------------------------------------------ entry points
def fp4_quantize(x, cfg, *, residual=None, outer=None, workspace=None, stream=None, out=None):
    """Rowwise quantisation of a bf16 or float32 x (views with any storage
    offset and row pitch are accepted).  Returns {"codes", "scales", "outer"}
    (outer None without a two-level mode).  `outer` is read when
    cfg.outer_mode == 1.  `out` may supply preallocated "codes" / "scales"."""
    torch = _torch()
    x, R, C, ld = _src(x, allow_f32=True)
    cfg = _with_dtypes(cfg, _dtype_name(x))
    dev = x.device
    sizes = fp4q_buffer_sizes(cfg, R, C)
    out = out or {}
    codes = out.get("codes")
    if codes is None:
        codes = _empty(sizes["row_codes"], torch.uint8, dev).view(R, C // 2)
    scales = out.get("scales")
    if scales is None:
        scales = _empty(sizes["row_scales"], torch.uint8, dev).view(R, C // _inner(cfg))
    if outer is None and sizes["row_outer"]:
        outer = _empty(sizes["row_outer"] // 4, torch.float32, dev)
    _need(codes, sizes["row_codes"], "codes")
    _need(scales, sizes["row_scales"], "scales")
    _need(outer, sizes["row_outer"], "outer")
    _need_residual(residual, R, C)
    ws, wsb = _workspace(cfg, R, C, dev, workspace)
    _check(lib().fp4_quantize(ct.byref(cfg), _ptr(x), R, C, ld, _ptr(codes), _ptr(scales), _ptr(outer),
                              _ptr(residual), _ptr(ws), wsb, _stream(stream)), "fp4_quantize")
    return {"codes": codes, "scales": scales, "outer": outer}


def fp4_qdq(x, cfg, *, residual=None, outer=None, with_codes=False, workspace=None, stream=None, y=None,
            y_dtype=None):
    """Quantise-dequantise rowwise (bf16 or float32 x; y in y_dtype, default
    x's dtype, or the dtype of a given y).  Returns {"y", "codes", "scales", "outer"}."""
    torch = _torch()
    x, R, C, ld = _src(x, allow_f32=True)
    dev = x.device
    if y is not None:
        y_dtype = y.dtype
    ydt = torch.float32 if (y_dtype if y_dtype is not None else x.dtype) == torch.float32 else torch.bfloat16
    cfg = _with_dtypes(cfg, _dtype_name(x), "fp32" if ydt == torch.float32 else "bf16")
    sizes = fp4q_buffer_sizes(cfg, R, C)
    if y is None:
        y = torch.empty((R, C), dtype=ydt, device=dev)
    codes = scales = None
    if with_codes:
        codes = _empty(sizes["row_codes"], torch.uint8, dev).view(R, C // 2)
        scales = _empty(sizes["row_scales"], torch.uint8, dev).view(R, C // _inner(cfg))
    if outer is None and sizes["row_outer"] and (with_codes or cfg.outer_mode == 0):
        outer = _empty(sizes["row_outer"] // 4, torch.float32, dev)
    _need(y, sizes["y"], "y")
    _need(outer, sizes["row_outer"], "outer")
    _need_residual(residual, R, C)
    ws, wsb = _workspace(cfg, R, C, dev, workspace)
    _check(lib().fp4_qdq(ct.byref(cfg), _ptr(x), R, C, ld, _ptr(y), _ptr(codes), _ptr(scales), _ptr(outer),
                         _ptr(residual), _ptr(ws), wsb, _stream(stream)), "fp4_qdq")
    return {"y": y, "codes": codes, "scales": scales, "outer": outer}


def fp4_qdq_noalloc(x, cfg, *, y, codes=None, scales=None, outer=None, residual=None, stream=None):
    """fp4_qdq without a workspace (the library's own per-GPU scratch), for
    callers that cannot allocate: every output tensor is passed in (y, and
    optionally codes, scales and outer), nothing is allocated here.  Calls that
    overlap on one GPU race.  Returns {"y", "codes", "scales", "outer"}."""
    x, R, C, ld = _src(x, allow_f32=True)
    cfg = _with_dtypes(cfg, _dtype_name(x), _dtype_name(y))
    sizes = fp4q_buffer_sizes(cfg, R, C)
    _need(y, sizes["y"], "y")
    _need(codes, sizes["row_codes"], "codes")
    _need(scales, sizes["row_scales"], "scales")
    _need(outer, sizes["row_outer"], "outer")
    _need_residual(residual, R, C)
    _check(lib().fp4_qdq_noalloc(ct.byref(cfg), _ptr(x), R, C, ld, _ptr(y), _ptr(codes), _ptr(scales), _ptr(outer),
                                 _ptr(residual), _stream(stream)), "fp4_qdq_noalloc")
    return {"y": y, "codes": codes, "scales": scales, "outer": outer}


def fp4_dequantize(codes, scales, outer, rows, cols, cfg, *, outer_transposed=False, stream=None, y=None,
                   dtype=None):
    """bf16 (or float32: dtype=torch.float32, or a float32 y) [rows, cols]
    from stored codes, scales and outer scales."""
    torch = _torch()
    if y is None:
        y = torch.empty((rows, cols), dtype=dtype if dtype is not None else torch.bfloat16, device=codes.device)
    cfg = _with_dtypes(cfg, output_dtype=_dtype_name(y))
    if rows and cols:
        sizes = fp4q_buffer_sizes(cfg, rows, cols)
        _need(codes, sizes["row_codes"], "codes")
        _need(scales, sizes["row_scales"], "scales")
        _need(outer, sizes["row_outer"], "outer")
        _need(y, sizes["y"], "y")
    _check(lib().fp4_dequantize(ct.byref(cfg), _ptr(codes), _ptr(scales), _ptr(outer), int(rows), int(cols),
                                int(bool(outer_transposed)), _ptr(y), _stream(stream)), "fp4_dequantize")
    return y


def fp4_cast_transpose(x, cfg, *, residual=None, row_outer=None, col_outer=None, workspace=None, stream=None,
                       out=None, staged=True):
    """Rowwise and columnwise buffers from one read of x.  Returns
    {"row_codes", "row_scales", "row_outer", "col_codes", "col_scales", "col_outer"}.
    `out` may supply any of the four code / scale tensors preallocated.
    Without a `workspace`, one is allocated: large enough to stage the outputs
    (staged=True) or only for the tensorwise scratch (staged=False)."""
    torch = _torch()
    x, R, C, ld = _src(x)
    dev = x.device
    sizes = fp4q_buffer_sizes(cfg, R, C)
    given = out or {}
    out = {
        "row_codes": given.get("row_codes"), "row_scales": given.get("row_scales"),
        "col_codes": given.get("col_codes"), "col_scales": given.get("col_scales"),
    }
    shapes = {"row_codes": (R, C // 2), "row_scales": (R, C // 16), "col_codes": (C, R // 2),
              "col_scales": (C, R // 16)}
    for k, shp in shapes.items():
        if out[k] is None:
            out[k] = _empty(shp[0] * shp[1], torch.uint8, dev).view(*shp)
    if row_outer is None and sizes["row_outer"]:
        row_outer = _empty(sizes["row_outer"] // 4, torch.float32, dev)
    if col_outer is None and sizes["col_outer"]:
        col_outer = _empty(sizes["col_outer"] // 4, torch.float32, dev)
    out["row_outer"], out["col_outer"] = row_outer, col_outer
    for k, shp in shapes.items():
        _need(out[k], shp[0] * shp[1], k)
    _need(row_outer, sizes["row_outer"], "row_outer")
    _need(col_outer, sizes["col_outer"], "col_outer")
    _need_residual(residual, R, C)
    ws, wsb = _ct_workspace(cfg, [R], C, residual, dev, workspace, staged)
    _check(lib().fp4_cast_transpose(ct.byref(cfg), _ptr(x), R, C, ld, _ptr(out["row_codes"]), _ptr(out["row_scales"]),
                                    _ptr(row_outer), _ptr(out["col_codes"]), _ptr(out["col_scales"]), _ptr(col_outer),
                                    _ptr(residual), _ptr(ws), wsb, _stream(stream)), "fp4_cast_transpose")
    return out


def fp4_cast_transpose_grouped(x, rows_per_group, cfg, *, residual=None, stream=None, out=None, workspace=None,
                               staged=True):
    """Per-group cast-transpose of groups stacked along rows (one launch per 64
    groups).  Returns flat stacked buffers (see include/fp4q.h).  `workspace`
    and `staged` as for fp4_cast_transpose."""
    torch = _torch()
    x, total, C, ld = _src(x)
    dev = x.device
    rows = [int(r) for r in rows_per_group]
    if sum(rows) != total:
        raise ValueError("rows_per_group does not sum to x.shape[0]")
    n_ro = n_co = 0
    for R in rows:
        s = fp4q_buffer_sizes(cfg, R, C)
        n_ro += s["row_outer"] // 4
        n_co += s["col_outer"] // 4
    if out is None:
        out = {
            "row_codes": _empty(total * C // 2, torch.uint8, dev).view(total, C // 2),
            "row_scales": _empty(total * C // 16, torch.uint8, dev).view(total, C // 16),
            "col_codes": _empty(total * C // 2, torch.uint8, dev),
            "col_scales": _empty(total * C // 16, torch.uint8, dev),
            "row_outer": _empty(n_ro, torch.float32, dev) if n_ro else None,
            "col_outer": _empty(n_co, torch.float32, dev) if n_co else None,
        }
    for k, n in (("row_codes", total * C // 2), ("row_scales", total * C // 16), ("col_codes", total * C // 2),
                 ("col_scales", total * C // 16), ("row_outer", 4 * n_ro), ("col_outer", 4 * n_co)):
        _need(out.get(k), n, k)
    _need_residual(residual, total, C)
    arr = (ct.c_int64 * max(len(rows), 1))(*rows)
    ws, wsb = _ct_workspace(cfg, rows, C, residual, dev, workspace, staged)
    _check(lib().fp4_cast_transpose_grouped(ct.byref(cfg), len(rows), arr, C, _ptr(x), ld, _ptr(out["row_codes"]),
                                            _ptr(out["row_scales"]), _ptr(out["row_outer"]), _ptr(out["col_codes"]),
                                            _ptr(out["col_scales"]), _ptr(out["col_outer"]), _ptr(residual), _ptr(ws),
                                            wsb, _stream(stream)), "fp4_cast_transpose_grouped")
    return out


def fp4_mx_project_fp8(x, cfg=None, *, y=True, mx8_row=True, mx8_col=True, blk=True, stream=None, out=None):
    """MXFP4 projection of x and its FP8 re-encodings in one pass.  Returns a
    dict with the requested outputs: "y" (bf16 [R, C]); "mx8_row" (uint8 E4M3
    [R, C]) and "mx8_row_scales" (uint8 UE8M0 [R, C/32]); "mx8_col" ([C, R]) and
    "mx8_col_scales" ([C, R/32]); "blk" ([R, C]), "blk_t" ([C, R]) and
    "blk_scales" (float32 [R/128, C/128]).  `out` may supply any of them."""
    torch = _torch()
    x, R, C, ld = _src(x)
    dev = x.device
    cfg = cfg if cfg is not None else make_cfg(format="mxfp4")
    out = dict(out or {})
    want = {"y": (y, (R, C), torch.bfloat16), "mx8_row": (mx8_row, (R, C), torch.uint8),
            "mx8_row_scales": (mx8_row, (R, C // 32), torch.uint8), "mx8_col": (mx8_col, (C, R), torch.uint8),
            "mx8_col_scales": (mx8_col, (C, R // 32), torch.uint8), "blk": (blk, (R, C), torch.uint8),
            "blk_t": (blk, (C, R), torch.uint8), "blk_scales": (blk, (R // 128, C // 128), torch.float32)}
    for k, (on, shp, dt) in want.items():
        if on and out.get(k) is None:
            out[k] = torch.empty(shp, dtype=dt, device=dev)
        if not on:
            out[k] = None
        else:
            _need(out[k], shp[0] * shp[1] * torch.empty((), dtype=dt).element_size(), k)
    g = out.get
    _check(lib().fp4_mx_project_fp8(ct.byref(cfg), _ptr(x), R, C, ld, _ptr(g("y")), _ptr(g("mx8_row")),
                                    _ptr(g("mx8_row_scales")), _ptr(g("mx8_col")), _ptr(g("mx8_col_scales")),
                                    _ptr(g("blk")), _ptr(g("blk_t")), _ptr(g("blk_scales")), _stream(stream)),
           "fp4_mx_project_fp8")
    return {k: v for k, v in out.items() if v is not None}


def fp4q_mx_scales_tiled_bytes(rows, K):
    return lib().fp4q_mx_scales_tiled_bytes(int(rows), int(K))


def fp4_mx_scales_tiled(scales, K, stream=None, out=None):
    """GEMM-ready layout of rowwise MXFP4 scales [rows, K/32] (uint8, flat)."""
    torch = _torch()
    rows = scales.shape[0]
    _need(scales, rows * (K // 32), "scales")
    if out is None:
        out = torch.empty(fp4q_mx_scales_tiled_bytes(rows, K), dtype=torch.uint8, device=scales.device)
    _need(out, fp4q_mx_scales_tiled_bytes(rows, K), "tiled scales")
    _check(lib().fp4_mx_scales_tiled(_ptr(scales), int(rows), int(K), _ptr(out), _stream(stream)),
           "fp4_mx_scales_tiled")
    return out


def fp4_mm(a, b, cfg=None, *, out_dtype=None, c=None, stream=None):
    """C = a @ b^T on the FP4 matrix cores with MXFP4 operands.  a ([M, K]) and
    b ([N, K]) are dicts {"codes", "scales"} as fp4_quantize returns them for
    MXFP4 (rowwise scales), or {"codes", "scales_tiled"} with GEMM-ready
    scales (fp4_mx_scales_tiled), or bf16 / float32 tensors, which are
    quantised and their scales tiled first.  C is bf16 unless out_dtype (or a
    given c) is float32."""
    torch = _torch()
    cfg = cfg if cfg is not None else make_cfg(format="mxfp4")

    def operand(x):
        if isinstance(x, dict):
            if "scales_tiled" in x:
                return x["codes"], x["scales_tiled"], 1
            return x["codes"], x["scales"], 0
        q = fp4_quantize(x, cfg, stream=stream)
        return q["codes"], fp4_mx_scales_tiled(q["scales"], x.shape[1], stream=stream), 1
    ac, asc, la = operand(a)
    bc, bsc, lb = operand(b)
    if la != lb:
        raise ValueError("both operands need the same scale layout")
    M, N, K = ac.shape[0], bc.shape[0], ac.shape[1] * 2
    if bc.shape[1] * 2 != K:
        raise ValueError("operands disagree on K (%d vs %d)" % (K, bc.shape[1] * 2))
    for nm, codes, sc, rows in (("a", ac, asc, M), ("b", bc, bsc, N)):
        _need(codes, rows * K // 2, nm + " codes")
        _need(sc, fp4q_mx_scales_tiled_bytes(rows, K) if la else rows * (K // 32), nm + " scales")
    if c is None:
        c = torch.empty((M, N), dtype=out_dtype if out_dtype is not None else torch.bfloat16, device=ac.device)
    if tuple(c.shape) != (M, N) or (N > 1 and c.stride(1) != 1) or c.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("c must be a bf16 or float32 [%d, %d] view with contiguous rows" % (M, N))
    ccfg = _with_dtypes(cfg, output_dtype=_dtype_name(c))
    _check(lib().fp4_mm(ct.byref(ccfg), _ptr(ac), _ptr(asc), _ptr(bc), _ptr(bsc), M, N, K, la, _ptr(c),
                        c.stride(0) if M > 1 else N, _stream(stream)), "fp4_mm")
    return c


class ErrorFeedback:
    """Per-tensor error-feedback state for quantised weights ("fp4-train"
    README, API: ErrorFeedback; Method: error feedback carries each step's
    quantisation error into the next step's value).

    One FP32 residual per name, created as zeros on the first call with the
    tensor's shape and device.  qdq(name, w, step) quantises RN(w + residual)
    and returns the dequantised tensor (w's dtype); the same kernel rewrites the
    residual in place with RN(value - dequantised value).  quantize() does the
    same and returns the packed codes and scales instead.  `step` is the
    stochastic-rounding counter of that call.  NVFP4 / AMD-FP4 only (MXFP4 has
    no error-feedback path).
    """

    def __init__(self, cfg=None, *, stochastic=False, seed=0, **cfg_kw):
        if cfg is None:
            cfg = make_cfg(rounding="stochastic" if stochastic else "rne", seed=seed, **cfg_kw)
        elif cfg_kw or stochastic or seed:
            raise ValueError("pass either cfg or its keyword settings, not both")
        if cfg.format == FORMATS["mxfp4"]:
            raise Fp4Error(ERR_UNSUPPORTED, "ErrorFeedback with MXFP4")
        self.cfg = cfg
        self._res = {}

    def _cfg(self, step):
        c = Cfg.from_buffer_copy(self.cfg)
        c.step = int(step)
        return c

    def residual(self, name, like=None):
        """The residual of `name` (created as zeros shaped like `like`)."""
        r = self._res.get(name)
        if r is None:
            if like is None:
                raise KeyError(name)
            torch = _torch()
            r = torch.zeros(like.shape, dtype=torch.float32, device=like.device)
            self._res[name] = r
        elif like is not None and (tuple(r.shape) != tuple(like.shape) or r.device != like.device):
            raise ValueError("residual of %r is %s on %s, tensor is %s on %s"
                             % (name, tuple(r.shape), r.device, tuple(like.shape), like.device))
        return r

    def qdq(self, name, w, step=0, **kw):
        return fp4_qdq(w, self._cfg(step), residual=self.residual(name, w), **kw)["y"]

    def quantize(self, name, w, step=0, **kw):
        return fp4_quantize(w, self._cfg(step), residual=self.residual(name, w), **kw)

    def reset(self, name=None):
        """Forget one residual (or all of them)."""
        if name is None:
            self._res.clear()
        else:
            self._res.pop(name, None)

    def state_dict(self):
        return {k: v.clone() for k, v in self._res.items()}

    def load_state_dict(self, state):
        torch = _torch()
        for k, v in state.items():
            if v.dtype != torch.float32 or v.dim() != 2:
                raise ValueError("residual %r must be a 2-D float32 tensor" % k)
        self._res = {k: v.clone().contiguous() for k, v in state.items()}
