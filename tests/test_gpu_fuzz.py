"""Seeded random configurations of the NV / AMD paths against the oracle.

Each case draws a format, a two-level mode (none, tensorwise, 1D outer groups
of 16 / 32 / 64 / 128, the 2D 64 x 64 outer tile), RNE or stochastic rounding
with a random seed, step and index base, an optional error-feedback residual,
an entry point (fp4_qdq, fp4_quantize, fp4_cast_transpose staged or direct,
fp4_cast_transpose_grouped), a shape with ragged tiles where the mode allows
them, and a source row pitch (a column-sliced view).  A second family draws
the remaining options: FP32 sources and FP32 outputs, outer scales supplied by
the caller, 16 x 16 inner tiles and MXFP4.  A third takes configurations of
the first kind and injects special values into the source and the residual.
Every output buffer is compared byte for byte with the oracle.  The draws are
fixed by the case number, so a failure names a reproducible case."""
import zlib

import numpy as np
import pytest
import torch

import block_scaled_fp4_amax_amd as fq
from block_scaled_fp4_amax_amd import workloads as W
from oracle import ref

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

N_CASES = 200
FMT = {"nvfp4": ("nvfp4", None, "e4m3"), "nvfp4-ue5m3": ("nvfp4", "ue5m3", "ue5m3"), "amdfp4": ("amdfp4", None, "ue5m3")}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fq.lib()


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def _host(t, dtype):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.detach().cpu().contiguous().numpy().view(dtype)


def _same(gpu, want, what):
    gpu, want = np.asarray(gpu), np.asarray(want)
    if want.dtype == np.float32:
        want, gpu = want.view(np.uint32), gpu.view(np.uint32)
    gpu = gpu.reshape(want.shape)
    bad = np.flatnonzero(gpu.ravel() != want.ravel())
    assert bad.size == 0, "%s: %d of %d differ; first at flat %d: gpu %s oracle %s" % (
        what, bad.size, want.size, bad[0], hex(int(gpu.ravel()[bad[0]])), hex(int(want.ravel()[bad[0]])))


def draw(case):
    rng = np.random.default_rng(1000 + case)
    c = {"fmt": str(rng.choice(list(FMT))), "sr": bool(rng.integers(2)), "ef": bool(rng.integers(2)),
         "seed": int(rng.integers(0, 2 ** 40)), "step": int(rng.integers(0, 1000)),
         "index_base": int(rng.integers(0, 2 ** 20)) * 8 + int(rng.integers(0, 8))}
    mode = str(rng.choice(["none", "tensorwise", "1d", "1d", "2d", "2d"]))
    c["op"] = str(rng.choice(["qdq", "quantize", "ct", "ct", "grouped"]))
    if mode == "2d":
        c.update(two_level="outer", obs=64, outer_2d=True)
        row_mult, col_mult = 64, 64          # both dimensions multiples of the 2D tile
    elif mode == "1d":
        obs = int(rng.choice([16, 32, 64, 128]))
        c.update(two_level="outer", obs=obs, outer_2d=False)
        row_mult, col_mult = (obs if c["op"] in ("ct", "grouped") else 16), obs
    else:
        c.update(two_level=mode, obs=0, outer_2d=False)
        row_mult, col_mult = 16, 16
    if c["op"] == "grouped" and mode == "tensorwise":
        mode = "none"
        c["two_level"] = "none"
    c["cols"] = col_mult * int(rng.integers(1, max(2, 400 // col_mult)))
    if c["op"] == "grouped":
        c["rows"] = [row_mult * int(rng.integers(0, max(2, 256 // row_mult))) for _ in range(int(rng.integers(1, 6)))]
        if sum(c["rows"]) == 0:
            c["rows"][0] = row_mult
    else:
        c["rows"] = row_mult * int(rng.integers(1, max(2, 320 // row_mult)))
    c["staged"] = bool(rng.integers(2))
    c["scale"] = float(rng.choice([1e-3, 0.02, 1.0, 300.0]))
    c["pad"] = int(rng.choice([0, 0, 8, 24, 64]))   # source row pitch cols + pad (a column-sliced view)
    return c


def _view(x, pad):
    """x on the device, as the first columns of a wider row-major tensor when
    pad > 0 (row pitch cols + pad)."""
    if pad == 0:
        return _dev(x)
    R, C = x.shape
    full = np.zeros((R, C + pad), np.uint16)
    full[:, :C] = x
    return _dev(full)[:, :C]


def _cfgs(c):
    f, sf, osf = FMT[c["fmt"]]
    gtl = {"none": "none", "tensorwise": "tensorwise", "outer": "outer_block"}[c["two_level"]]
    g = fq.make_cfg(format=f, scale_format=sf, two_level=gtl, outer_block_size=c["obs"], outer_2d=c["outer_2d"],
                    rounding="stochastic" if c["sr"] else "rne", seed=c["seed"], step=c["step"],
                    index_base=c["index_base"])
    o = dict(scale_fmt=osf, two_level=c["two_level"], obs=c["obs"], outer_2d=c["outer_2d"], stochastic=c["sr"],
             seed=c["seed"], step=c["step"], index_base=c["index_base"])
    return g, o


@pytest.mark.parametrize("case", range(N_CASES), ids=lambda i: "fuzz-%d" % i)
def test_random_configuration_matches_oracle(case):
    c = draw(case)
    rng = np.random.default_rng(zlib.crc32(repr(c).encode()))
    R = sum(c["rows"]) if c["op"] == "grouped" else c["rows"]
    C = c["cols"]
    a = rng.standard_normal((R, C)).astype(np.float32) * np.float32(c["scale"])
    a *= np.exp(rng.standard_normal((R, 1))).astype(np.float32)
    x = W.to_bf16(a)
    z0 = (rng.standard_normal((R, C)) * 0.01 * c["scale"]).astype(np.float32) if c["ef"] else None
    g, o = _cfgs(c)
    zo = None if z0 is None else z0.copy()
    zd = None if z0 is None else torch.from_numpy(z0.copy()).cuda()
    what = repr(c)
    if c["op"] in ("qdq", "quantize"):
        want = ref.nv_quantize(x, residual=zo, **o)
        if c["op"] == "qdq":
            out = fq.fp4_qdq(_view(x, c["pad"]), g, residual=zd, with_codes=True)
            _same(_host(out["y"], np.uint16), want["row_y"], what + " y")
        else:
            out = fq.fp4_quantize(_view(x, c["pad"]), g, residual=zd)
        _same(_host(out["codes"], np.uint8), want["row_codes"], what + " codes")
        _same(_host(out["scales"], np.uint8), want["row_scales"], what + " scales")
        if "row_outer" in want:
            _same(_host(out["outer"], np.float32), want["row_outer"], what + " outer")
    elif c["op"] == "ct":
        want = ref.nv_quantize(x, residual=zo, cols=True, want_y=False, **o)
        out = fq.fp4_cast_transpose(_view(x, c["pad"]), g, residual=zd, staged=c["staged"])
        for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
            _same(_host(out[k], np.uint8), want[k], what + " " + k)
        for k in ("row_outer", "col_outer"):
            if k in want:
                _same(_host(out[k], np.float32), want[k], what + " " + k)
    else:
        want = ref.nv_quantize_grouped(x, c["rows"], residual=zo, **o)
        out = fq.fp4_cast_transpose_grouped(_view(x, c["pad"]), c["rows"], g, residual=zd, staged=c["staged"])
        for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
            _same(_host(out[k], np.uint8).reshape(want[k].shape), want[k], what + " " + k)
        for k in ("row_outer", "col_outer"):
            w = np.asarray(want.get(k, np.zeros(0, np.float32)), np.float32).ravel()
            if out.get(k) is None:
                assert w.size == 0, what + " " + k + ": the oracle has outer scales, the call returned none"
            else:
                _same(_host(out[k], np.float32).ravel(), w, what + " " + k)
    if c["ef"]:
        _same(_host(zd, np.float32), zo, what + " residual")


# ------------------------------------------------------------------ more options
N_MORE = 120


def draw_more(case):
    """FP32 sources and FP32 targets (rowwise entry points), precomputed outer
    scales (outer_mode 1, no residual), 16 x 16 inner tiles, and MXFP4."""
    rng = np.random.default_rng(5000 + case)
    kind = str(rng.choice(["f32", "given", "inner2d", "mx"]))
    c = {"kind": kind, "fmt": str(rng.choice(list(FMT))), "sr": bool(rng.integers(2)),
         "seed": int(rng.integers(0, 2 ** 40)), "step": int(rng.integers(0, 1000)),
         "index_base": int(rng.integers(0, 2 ** 20)) * 8 + int(rng.integers(0, 8)),
         "scale": float(rng.choice([1e-3, 0.02, 1.0, 300.0])), "ef": False, "obs": 0, "outer_2d": False}
    if kind == "f32":
        mode = str(rng.choice(["none", "tensorwise", "1d"]))
        c["op"] = str(rng.choice(["qdq", "quantize"]))
        c["ef"] = bool(rng.integers(2))
        c["y_f32"] = bool(rng.integers(2))
        if mode == "1d":
            c.update(two_level="outer", obs=int(rng.choice([16, 32, 64, 128])))
        else:
            c["two_level"] = mode
        c["rows"] = 16 * int(rng.integers(1, 20))
        c["cols"] = max(16, c["obs"]) * int(rng.integers(1, max(2, 320 // max(16, c["obs"]))))
    elif kind == "given":
        o2d = bool(rng.integers(2))
        c["op"] = str(rng.choice(["quantize", "ct"]))
        obs = 64 if o2d else int(rng.choice([16, 32, 64]))
        c.update(two_level="outer", obs=obs, outer_2d=o2d)
        c["rows"] = (64 if o2d or c["op"] == "ct" else 16) * int(rng.integers(1, 5))
        c["cols"] = obs * int(rng.integers(1, max(2, 320 // obs)))
    elif kind == "inner2d":
        mode = str(rng.choice(["none", "tensorwise", "2d"]))
        c["op"] = str(rng.choice(["quantize", "ct"]))
        c["ef"] = bool(rng.integers(2))
        if mode == "2d":
            c.update(two_level="outer", obs=64, outer_2d=True)
            c["rows"], c["cols"] = 64 * int(rng.integers(1, 5)), 64 * int(rng.integers(1, 5))
        else:
            c["two_level"] = mode
            c["rows"], c["cols"] = 16 * int(rng.integers(1, 17)), 16 * int(rng.integers(1, 21))
    else:
        c["op"] = str(rng.choice(["qdq", "quantize"]))
        c["y_f32"] = bool(rng.integers(2))
        c["x_f32"] = bool(rng.integers(2))
        c["rows"], c["cols"] = int(rng.integers(1, 80)), 32 * int(rng.integers(1, 12))
    return c


@pytest.mark.parametrize("case", range(N_MORE), ids=lambda i: "more-%d" % i)
def test_random_option_matches_oracle(case):
    c = draw_more(case)
    rng = np.random.default_rng(zlib.crc32(repr(c).encode()))
    R, C = c["rows"], c["cols"]
    a = rng.standard_normal((R, C)).astype(np.float32) * np.float32(c["scale"])
    a *= np.exp(rng.standard_normal((R, 1))).astype(np.float32)
    what = repr(c)
    if c["kind"] == "mx":
        x = a if c["x_f32"] else W.to_bf16(a)
        ydt = "fp32" if c["y_f32"] else "bf16"
        codes, scales, y = ref.mx_qdq(x, y_dtype=ydt)
        g = fq.make_cfg(format="mxfp4")
        xd = torch.from_numpy(x).cuda() if c["x_f32"] else _dev(x)
        if c["op"] == "qdq":
            out = fq.fp4_qdq(xd, g, with_codes=True, y_dtype=torch.float32 if c["y_f32"] else torch.bfloat16)
            _same(_host(out["y"], np.float32 if c["y_f32"] else np.uint16), y, what + " y")
        else:
            out = fq.fp4_quantize(xd, g)
        _same(_host(out["codes"], np.uint8), codes, what + " codes")
        _same(_host(out["scales"], np.uint8), scales, what + " scales")
        return
    g, o = _cfgs(c)
    if c["kind"] == "f32":
        x = a
        xd = torch.from_numpy(x).cuda()
    else:
        x = W.to_bf16(a)
        xd = _dev(x)
    z0 = (rng.standard_normal((R, C)) * 0.01 * c["scale"]).astype(np.float32) if c["ef"] else None
    zo = None if z0 is None else z0.copy()
    zd = None if z0 is None else torch.from_numpy(z0.copy()).cuda()
    if c["kind"] == "inner2d":
        g.inner_2d = 1
        o["inner_2d"] = True
    if c["kind"] == "given":
        natural = ref.nv_quantize(x, cols=c["op"] == "ct", want_y=False, **o)
        row_o = natural["row_outer"] * np.float32(rng.uniform(0.5, 2.0))
        col_o = natural.get("col_outer")
        col_o = None if col_o is None else col_o * np.float32(rng.uniform(0.5, 2.0))
        g.outer_mode = 1
        want = ref.nv_quantize(x, cols=c["op"] == "ct", want_y=False, given_outer=(row_o, col_o), **o)
        ro = torch.from_numpy(np.ascontiguousarray(row_o, np.float32)).cuda()
        co = None if col_o is None else torch.from_numpy(np.ascontiguousarray(col_o, np.float32)).cuda()
        if c["op"] == "ct":
            out = fq.fp4_cast_transpose(xd, g, row_outer=ro, col_outer=co)
            for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
                _same(_host(out[k], np.uint8), want[k], what + " " + k)
        else:
            out = fq.fp4_quantize(xd, g, outer=ro)
            _same(_host(out["codes"], np.uint8), want["row_codes"], what + " codes")
            _same(_host(out["scales"], np.uint8), want["row_scales"], what + " scales")
        return
    if c["op"] == "ct":
        want = ref.nv_quantize(x, residual=zo, cols=True, want_y=False, **o)
        out = fq.fp4_cast_transpose(xd, g, residual=zd)
        for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
            _same(_host(out[k], np.uint8), want[k], what + " " + k)
    elif c["op"] == "qdq":
        ydt = "fp32" if c.get("y_f32") else "bf16"
        want = ref.nv_quantize(x, residual=zo, y_dtype=ydt, **o)
        out = fq.fp4_qdq(xd, g, residual=zd, with_codes=True,
                         y_dtype=torch.float32 if ydt == "fp32" else torch.bfloat16)
        _same(_host(out["y"], np.float32 if ydt == "fp32" else np.uint16), want["row_y"], what + " y")
        _same(_host(out["codes"], np.uint8), want["row_codes"], what + " codes")
        _same(_host(out["scales"], np.uint8), want["row_scales"], what + " scales")
    else:
        want = ref.nv_quantize(x, residual=zo, want_y=False, **o)
        out = fq.fp4_quantize(xd, g, residual=zd)
        _same(_host(out["codes"], np.uint8), want["row_codes"], what + " codes")
        _same(_host(out["scales"], np.uint8), want["row_scales"], what + " scales")
    if "row_outer" in want and out.get("outer" if c["op"] != "ct" else "row_outer") is not None:
        _same(_host(out["outer" if c["op"] != "ct" else "row_outer"], np.float32), want["row_outer"], what + " outer")
    if c["ef"]:
        _same(_host(zd, np.float32), zo, what + " residual")


# ------------------------------------------------------------------ special values
N_EDGE = 120
_SPECIAL_BF16 = np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x7F81, 0x0001, 0x8001, 0x007F,
                          0x807F, 0x0080, 0x7F7F, 0xFF7F, 0x7F7E], np.uint16)


def _inject(x, rng, density):
    """bf16 bits with specials: zeros, infinities, NaNs, subnormals, the
    largest finite values, E2M1 decision points and grid values times random
    powers of two (and one ulp either side), and constant or zero 16-blocks."""
    x = x.copy()
    R, C = x.shape
    n = max(1, int(density * R * C))
    pos = rng.integers(0, R * C, size=n)
    kind = rng.integers(0, 3, size=n)
    flat = x.ravel()
    sp = _SPECIAL_BF16[rng.integers(0, _SPECIAL_BF16.size, size=n)]
    grid = W.MID_VALUES[rng.integers(0, W.MID_VALUES.size, size=n)] * np.exp2(rng.integers(-30, 31, size=n)).astype(np.float32)
    gb = W.to_bf16(grid * np.where(rng.random(n) < 0.5, -1, 1).astype(np.float32))
    gb = (gb.astype(np.int32) + rng.integers(-1, 2, size=n)).astype(np.uint16)
    flat[pos] = np.where(kind == 0, sp, gb)
    for _ in range(max(1, R * C // 2048)):           # whole 16-blocks: one constant, or zero
        r, b = int(rng.integers(0, R)), int(rng.integers(0, C // 16))
        flat[r * C + 16 * b: r * C + 16 * b + 16] = 0 if rng.random() < 0.5 else flat[r * C + 16 * b]
    return x


def _inject_residual(z, rng, density):
    """Finite residual specials: signed zeros, binary32 subnormals, values near
    the largest finite binary32 (so that x + r overflows)."""
    z = z.copy()
    n = max(1, int(density * z.size))
    pos = rng.integers(0, z.size, size=n)
    vals = np.array([0.0, -0.0, 1e-45, -1e-45, 1e-40, 3e38, -3e38, 3.4e38], np.float32)
    z.ravel()[pos] = vals[rng.integers(0, vals.size, size=n)]
    return z


@pytest.mark.parametrize("case", range(N_EDGE), ids=lambda i: "edge-%d" % i)
def test_random_configuration_with_special_values(case):
    c = draw(9000 + case)
    rng = np.random.default_rng(zlib.crc32(("edge" + repr(c)).encode()))
    R = sum(c["rows"]) if c["op"] == "grouped" else c["rows"]
    C = c["cols"]
    a = rng.standard_normal((R, C)).astype(np.float32) * np.float32(c["scale"])
    a *= np.exp(rng.standard_normal((R, 1))).astype(np.float32)
    density = float(rng.choice([0.002, 0.02, 0.1]))
    x = _inject(W.to_bf16(a), rng, density)
    z0 = None
    if c["ef"]:
        z0 = _inject_residual((rng.standard_normal((R, C)) * 0.01 * c["scale"]).astype(np.float32), rng, density)
    g, o = _cfgs(c)
    zo = None if z0 is None else z0.copy()
    zd = None if z0 is None else torch.from_numpy(z0.copy()).cuda()
    what = repr(c) + " density %g" % density
    if c["op"] in ("qdq", "quantize"):
        want = ref.nv_quantize(x, residual=zo, **o)
        if c["op"] == "qdq":
            out = fq.fp4_qdq(_view(x, c["pad"]), g, residual=zd, with_codes=True)
            _same(_host(out["y"], np.uint16), want["row_y"], what + " y")
        else:
            out = fq.fp4_quantize(_view(x, c["pad"]), g, residual=zd)
        _same(_host(out["codes"], np.uint8), want["row_codes"], what + " codes")
        _same(_host(out["scales"], np.uint8), want["row_scales"], what + " scales")
        if "row_outer" in want:
            _same(_host(out["outer"], np.float32), want["row_outer"], what + " outer")
    elif c["op"] == "ct":
        want = ref.nv_quantize(x, residual=zo, cols=True, want_y=False, **o)
        out = fq.fp4_cast_transpose(_view(x, c["pad"]), g, residual=zd, staged=c["staged"])
        for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
            _same(_host(out[k], np.uint8), want[k], what + " " + k)
        for k in ("row_outer", "col_outer"):
            if k in want:
                _same(_host(out[k], np.float32), want[k], what + " " + k)
    else:
        want = ref.nv_quantize_grouped(x, c["rows"], residual=zo, **o)
        out = fq.fp4_cast_transpose_grouped(_view(x, c["pad"]), c["rows"], g, residual=zd, staged=c["staged"])
        for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
            _same(_host(out[k], np.uint8).reshape(want[k].shape), want[k], what + " " + k)
        for k in ("row_outer", "col_outer"):
            w = np.asarray(want.get(k, np.zeros(0, np.float32)), np.float32).ravel()
            if out.get(k) is None:
                assert w.size == 0, what + " " + k
            else:
                _same(_host(out[k], np.float32).ravel(), w, what + " " + k)
    if c["ef"]:
        _same(_host(zd, np.float32), zo, what + " residual")
