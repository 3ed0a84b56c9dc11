"""The staged cast-transpose (calls with an error-feedback residual: outputs
written as whole lines through a tile-major scratch and a gather pass) against
the oracle and against the direct-store path, bit for bit, on ragged shapes
(rows and columns that are not multiples of 64), scale buffers at odd
addresses (the unaligned gather), every outer kind, the tensorwise scratch
beside the staged region, and grouped calls that take several launches."""
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
    return t.detach().cpu().contiguous().numpy().view(dtype)


def same(gpu, want, what):
    gpu, want = np.asarray(gpu), np.asarray(want)
    if want.dtype == np.float32:
        want, gpu = want.view(np.uint32), gpu.view(np.uint32)
    gpu = gpu.reshape(want.shape)
    bad = np.flatnonzero(gpu.ravel() != want.ravel())
    assert bad.size == 0, "%s: %d of %d differ; first at flat %d: gpu %s want %s" % (
        what, bad.size, want.size, bad[0], hex(int(gpu.ravel()[bad[0]])), hex(int(want.ravel()[bad[0]])))


def rand_bf16(rng, shape, scale=0.02):
    a = rng.standard_normal(shape).astype(np.float32) * np.float32(scale)
    a *= np.exp(rng.standard_normal((shape[0], 1))).astype(np.float32)
    return W.to_bf16(a)


FMT = {"nvfp4": "e4m3", "amdfp4": "ue5m3"}
CASES = [
    # fmt, two_level, obs, outer_2d, sr, shape (all with an error-feedback residual: the calls that stage)
    ("nvfp4", "outer", 64, True, True, (192, 320)),
    ("nvfp4", "outer", 64, True, False, (128, 2880)),
    ("amdfp4", "outer", 64, False, True, (256, 2880)),
    ("amdfp4", "outer", 32, False, True, (96, 160)),
    ("nvfp4", "outer", 16, False, False, (48, 80)),
    ("nvfp4", "none", 0, False, True, (144, 208)),
    ("nvfp4", "none", 0, False, False, (80, 48)),
    ("nvfp4", "tensorwise", 0, False, True, (112, 96)),
    ("amdfp4", "tensorwise", 0, False, False, (64, 64)),
    ("nvfp4", "outer", 64, False, False, (320, 192)),
    ("amdfp4", "outer", 128, False, True, (256, 384)),
    # whole 64-column tiles with 1D outer groups of 32 and 16: the gather's
    # outer-scale runs of 8 and 16 bytes per tile line take its run-copy path
    ("amdfp4", "outer", 32, False, True, (128, 192)),
    ("nvfp4", "outer", 16, False, True, (64, 256)),
    ("nvfp4", "outer", 32, False, False, (96, 128)),
]


def _run(x, cfg, residual, staged, scale_offset=0):
    R, C = x.shape
    out = None
    if scale_offset:
        # scale buffers starting scale_offset bytes into an allocation
        rs = torch.full((R * C // 16 + 16,), 0xA5, dtype=torch.uint8, device="cuda")[scale_offset:scale_offset + R * C // 16]
        cs = torch.full((R * C // 16 + 16,), 0xA5, dtype=torch.uint8, device="cuda")[scale_offset:scale_offset + R * C // 16]
        out = {"row_scales": rs.view(R, C // 16), "col_scales": cs.view(C, R // 16)}
    return fq.fp4_cast_transpose(dev(x), cfg, residual=residual, staged=staged, out=out)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(str(v) for v in c[:5]) + "-%dx%d" % c[5])
def test_staged_equals_oracle_and_direct(case):
    fmt, tl, obs, o2d, sr, shape = case
    R, C = shape
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    x = rand_bf16(rng, shape)
    x[:, rng.integers(0, C)] = W.to_bf16(W.from_bf16(x[:, 0]) * np.float32(800))
    z0 = (rng.standard_normal(shape) * 0.003).astype(np.float32)
    gtl = {"none": "none", "tensorwise": "tensorwise", "outer": "outer_block"}[tl]
    cfg = fq.make_cfg(format=fmt, two_level=gtl, outer_block_size=obs, outer_2d=o2d,
                      rounding="stochastic" if sr else "rne", seed=17, step=2)
    zo = z0.copy()
    want = ref.nv_quantize(x, scale_fmt=FMT[fmt], two_level=tl, obs=obs, outer_2d=o2d, stochastic=sr, seed=17, step=2,
                           residual=zo, cols=True, want_y=False)
    # a residual makes the call stage; without one the query holds only the tensorwise scratch
    no_res = fq.fp4q_cast_transpose_workspace_bytes(cfg, [R], C, False)
    assert no_res >= fq.fp4q_workspace_bytes(cfg, R, C) and (no_res > 0) == (tl == "tensorwise")
    assert fq.fp4q_cast_transpose_workspace_bytes(cfg, [R], C, True) > no_res
    for staged, off in ((True, 0), (True, 1), (False, 0)):
        zd = torch.from_numpy(z0.copy()).cuda()
        out = _run(x, cfg, zd, staged, off)
        for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
            same(host(out[k], np.uint8), want[k], "staged=%s off=%d %s" % (staged, off, k))
        for k in ("row_outer", "col_outer"):
            if k in want:
                same(host(out[k], np.float32), want[k], "staged=%s %s" % (staged, k))
        same(host(zd, np.float32), zo, "staged=%s residual" % staged)


@pytest.mark.parametrize("tl,obs,o2d", [("outer", 64, True), ("outer", 32, False), ("none", 0, False)])
def test_staged_grouped_many_groups(tl, obs, o2d):
    rng = np.random.default_rng(77 + obs)
    step = 64 if o2d or obs == 64 else 32 if obs == 32 else 16
    rows = [int(v) for v in rng.choice([0, step, 2 * step, 5 * step], size=97)]
    C = 192
    x = rand_bf16(rng, (sum(rows), C))
    z0 = (rng.standard_normal(x.shape) * 0.01).astype(np.float32)
    gtl = {"outer": "outer_block", "none": "none"}[tl]
    g = fq.make_cfg(format="nvfp4", two_level=gtl, outer_block_size=obs, outer_2d=o2d, rounding="stochastic",
                    seed=23, step=6, index_base=8)
    zo = z0.copy()
    want = ref.nv_quantize_grouped(x, rows, two_level=tl, obs=obs, outer_2d=o2d, stochastic=True, seed=23, step=6,
                                   index_base=8, residual=zo)
    for staged in (True, False):
        zd = torch.from_numpy(z0.copy()).cuda()
        out = fq.fp4_cast_transpose_grouped(dev(x), rows, g, residual=zd, staged=staged)
        for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
            same(host(out[k], np.uint8).reshape(want[k].shape), want[k], "staged=%s %s" % (staged, k))
        if tl == "outer":
            same(host(out["row_outer"], np.float32).ravel(), want["row_outer"], "staged=%s row outer" % staged)
        if tl == "outer" and not o2d:
            same(host(out["col_outer"], np.float32).ravel(), want["col_outer"], "staged=%s col outer" % staged)
        same(host(zd, np.float32), zo, "staged=%s residual" % staged)


def test_staged_full_size_1d_sr_ef_16384x2880():
    """The 16384 x 2880 activation workload's configuration (AMD-FP4 1D 1x64
    outer, SR) with an error-feedback residual, so it stages: every buffer and
    the residual against the oracle."""
    x = W.activations_16384x2880()
    R, C = x.shape
    cfg = fq.make_cfg(format="amdfp4", two_level="outer_block", outer_block_size=64, rounding="stochastic", seed=7,
                      step=3)
    z0 = (np.random.default_rng(41).standard_normal((R, C)) * 0.05).astype(np.float32)
    zo = z0.copy()
    want = ref.nv_quantize(x, scale_fmt="ue5m3", two_level="outer", obs=64, stochastic=True, seed=7, step=3,
                           residual=zo, cols=True, want_y=False)
    zd = torch.from_numpy(z0).cuda()
    out = fq.fp4_cast_transpose(dev(x), cfg, residual=zd, staged=True)
    for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
        same(host(out[k], np.uint8), want[k], "staged 16384x2880 " + k)
    for k in ("row_outer", "col_outer"):
        same(host(out[k], np.float32), want[k], "staged 16384x2880 " + k)
    same(host(zd, np.float32), zo, "staged 16384x2880 residual")
