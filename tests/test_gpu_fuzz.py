"""Seeded random configurations of the NV / AMD paths against the oracle.

Each case draws a format, a two-level mode (none, tensorwise, 1D outer groups
of 16 / 32 / 64 / 128, the 2D 64 x 64 outer tile), RNE or stochastic rounding
with a random seed, step and index base, an optional error-feedback residual,
an entry point (fp4_qdq, fp4_quantize, fp4_cast_transpose staged or direct,
fp4_cast_transpose_grouped) and a shape with ragged tiles where the mode allows
them.  Every output buffer is compared byte for byte with the oracle.  The
draws are fixed by the case number, so a failure names a reproducible case."""
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
    return c


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
            out = fq.fp4_qdq(_dev(x), g, residual=zd, with_codes=True)
            _same(_host(out["y"], np.uint16), want["row_y"], what + " y")
        else:
            out = fq.fp4_quantize(_dev(x), g, residual=zd)
        _same(_host(out["codes"], np.uint8), want["row_codes"], what + " codes")
        _same(_host(out["scales"], np.uint8), want["row_scales"], what + " scales")
        if "row_outer" in want:
            _same(_host(out["outer"], np.float32), want["row_outer"], what + " outer")
    elif c["op"] == "ct":
        want = ref.nv_quantize(x, residual=zo, cols=True, want_y=False, **o)
        out = fq.fp4_cast_transpose(_dev(x), g, residual=zd, staged=c["staged"])
        for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
            _same(_host(out[k], np.uint8), want[k], what + " " + k)
        for k in ("row_outer", "col_outer"):
            if k in want:
                _same(_host(out[k], np.float32), want[k], what + " " + k)
    else:
        want = ref.nv_quantize_grouped(x, c["rows"], residual=zo, **o)
        out = fq.fp4_cast_transpose_grouped(_dev(x), c["rows"], g, residual=zd, staged=c["staged"])
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
