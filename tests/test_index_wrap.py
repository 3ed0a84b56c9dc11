"""Stochastic-rounding indices that wrap past 2^64.

Element (i, j) draws its variate at index index_base + i * cols + j taken
modulo 2^64 (the header's definition of index_base; the oracle forms it in
uint64 arithmetic, "fp4-train" README, Method: one counter-based variate per
element).  Each case puts the wrap inside the tensor: in the middle of a
16-block of the first row, at the start of a later tile row, and inside the
second group of a grouped call.  Every output buffer is compared byte for
byte with the oracle."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_amax_amd as fq
from block_scaled_fp4_amax_amd import workloads as W
from oracle import ref

TOP = 1 << 64
SEED, STEP = 0xC0FFEE1234, 9


@pytest.fixture(scope="module")
def dev():
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


def _data(R, C, seed):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((R, C)).astype(np.float32) * np.exp(rng.standard_normal((R, 1))).astype(np.float32)
    return W.to_bf16(a), (rng.standard_normal((R, C)) * 0.01).astype(np.float32)


def test_wrapped_indices_draw_the_wrapped_variates():
    """(CPU) The oracle's variates at index_base + e are those at the wrapped index."""
    base = TOP - 5
    u = ref.sr_u16_array(SEED, STEP, base, 16)
    want = np.array([ref.sr_u16(SEED, STEP, (base + k) % TOP) for k in range(16)], np.uint16)
    assert (u == want).all()
    assert (u[5:] == ref.sr_u16_array(SEED, STEP, 0, 11)).all()


ROW_CASES = [
    # (format, two_level, obs, shape, index_base)
    ("nvfp4", "outer", 64, (64, 256), TOP - 37),            # the wrap inside a 16-block of row 0
    ("amdfp4", "outer", 16, (48, 128), TOP - 128 * 20),       # at the start of row 20
    ("nvfp4", "tensorwise", 0, (256, 256), TOP - 1000),      # the one-launch tensorwise path
    ("nvfp4", "none", 0, (1024, 1024), TOP - 3 * 1024 - 8),  # at element 8 of row 3, two-pass path
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", ROW_CASES, ids=lambda c: "%s-%s-%d-%dx%d" % (c[0], c[1], c[2], *c[3]))
@pytest.mark.parametrize("op", ["quantize", "qdq"])
def test_rowwise(dev, case, op):
    fmt, tl, obs, (R, C), base = case
    x, _ = _data(R, C, 11)
    g = fq.make_cfg(format=fmt, two_level={"outer": "outer_block"}.get(tl, tl), outer_block_size=obs,
                    rounding="stochastic", seed=SEED, step=STEP, index_base=base)
    kw = dict(scale_fmt="e4m3" if fmt == "nvfp4" else "ue5m3", two_level=tl, obs=obs, stochastic=True, seed=SEED,
              step=STEP, index_base=base)
    if op == "qdq":
        want = ref.nv_quantize(x, **kw)
        out = fq.fp4_qdq(_dev(x), g, with_codes=True)
        _same(_host(out["y"], np.uint16), want["row_y"], "y")
    else:
        want = ref.nv_quantize(x, want_y=False, **kw)
        out = fq.fp4_quantize(_dev(x), g)
    _same(_host(out["codes"], np.uint8), want["row_codes"], "codes")
    _same(_host(out["scales"], np.uint8), want["row_scales"], "scales")


CT_CASES = [
    # (format, mode, shape, index_base, residual)
    ("nvfp4", "2d", (128, 192), TOP - 64 * 192 - 5, True),       # inside row 64, the second tile row
    ("nvfp4", "2d", (128, 192), TOP - 64 * 192 - 5, False),
    ("amdfp4", "1d", (128, 128), TOP - 3, True),
    ("amdfp4", "1d", (128, 128), TOP - 3, False),
    ("nvfp4", "none", (64, 128), TOP - 100, True),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", CT_CASES, ids=lambda c: "%s-%s-%dx%d-%s" % (c[0], c[1], *c[2], "ef" if c[4] else "no-ef"))
@pytest.mark.parametrize("staged", [True, False])
def test_cast_transpose(dev, case, staged):
    fmt, mode, (R, C), base, ef = case
    x, z = _data(R, C, 12)
    tl = "none" if mode == "none" else "outer"
    kw = dict(scale_fmt="e4m3" if fmt == "nvfp4" else "ue5m3", two_level=tl, obs=0 if tl == "none" else 64,
              outer_2d=mode == "2d", stochastic=True, seed=SEED, step=STEP, index_base=base)
    g = fq.make_cfg(format=fmt, two_level="none" if tl == "none" else "outer_block", outer_block_size=kw["obs"],
                    outer_2d=mode == "2d", rounding="stochastic", seed=SEED, step=STEP, index_base=base)
    zo = z.copy() if ef else None
    zd = torch.from_numpy(z.copy()).cuda() if ef else None
    want = ref.nv_quantize(x, residual=zo, cols=True, want_y=False, **kw)
    out = fq.fp4_cast_transpose(_dev(x), g, residual=zd, staged=staged)
    for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
        _same(_host(out[k], np.uint8), want[k], k)
    for k in ("row_outer", "col_outer"):
        if k in want:
            _same(_host(out[k], np.float32), want[k], k)
    if ef:
        _same(_host(zd, np.float32), zo, "residual")


@pytest.mark.gpu
@pytest.mark.parametrize("staged", [True, False])
def test_grouped_wrap_in_second_group(dev, staged):
    rows = [64, 128]
    C = 128
    base = TOP - 64 * C - 70        # group 1 starts at element 64 * C: the wrap falls in its first row
    x, z = _data(sum(rows), C, 13)
    kw = dict(scale_fmt="e4m3", two_level="outer", obs=64, outer_2d=True, stochastic=True, seed=SEED, step=STEP,
              index_base=base)
    g = fq.make_cfg(format="nvfp4", two_level="outer_block", outer_block_size=64, outer_2d=True,
                    rounding="stochastic", seed=SEED, step=STEP, index_base=base)
    zo = z.copy()
    zd = torch.from_numpy(z.copy()).cuda()
    want = ref.nv_quantize_grouped(x, rows, residual=zo, **kw)
    out = fq.fp4_cast_transpose_grouped(_dev(x), rows, g, residual=zd, staged=staged)
    for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
        _same(_host(out[k], np.uint8).reshape(want[k].shape), want[k], k)
    _same(_host(out["row_outer"], np.float32).ravel(), want["row_outer"].ravel(), "row_outer")
    _same(_host(zd, np.float32), zo, "residual")
