"""Large tensors: output buffers beyond 4 GiB, up to the shape limit.

The kernels index inside a tile or a row with 32-bit offsets and form every
base in 64-bit arithmetic; the entry points refuse shapes whose element count
reaches 2^34.  These cases generate their input on the device and compare
64-row bands (the first, one in the middle and the last) with the oracle run
on the same band, with the band's global SR index base, so every output byte of
those bands is checked where the offsets are largest."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_amax_amd as fq
from oracle import ref

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fq.lib()
    yield
    torch.cuda.empty_cache()


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


def _bands(R):
    return [0, (R // 2) // 64 * 64, R - 64]


def _source(R, C, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn((R, C), generator=g, device="cuda", dtype=torch.bfloat16)
    x.mul_(0.25)
    return x


def test_rowwise_near_the_element_limit():
    """fp4_quantize, NVFP4 with 1D outer groups of 64 and stochastic rounding,
    (2^20 - 64) x 16384 bf16: 2^34 - 2^20 elements (the limit is 2^34), 32 GiB
    in, 8 GiB of codes."""
    R, C = (1 << 20) - 64, 16384
    base = 12345
    x = _source(R, C, 1)
    cfg = fq.make_cfg(format="nvfp4", two_level="outer_block", outer_block_size=64, rounding="stochastic",
                      seed=77, step=5, index_base=base)
    out = fq.fp4_quantize(x, cfg)
    torch.cuda.synchronize()
    for r0 in _bands(R):
        xb = _host(x[r0:r0 + 64], np.uint16)
        want = ref.nv_quantize(xb, scale_fmt="e4m3", two_level="outer", obs=64, stochastic=True, seed=77, step=5,
                               index_base=base + r0 * C, want_y=False)
        _same(_host(out["codes"][r0:r0 + 64], np.uint8), want["row_codes"], "codes rows %d.." % r0)
        _same(_host(out["scales"][r0:r0 + 64], np.uint8), want["row_scales"], "scales rows %d.." % r0)
        _same(_host(out["outer"].view(R, C // 64)[r0:r0 + 64], np.float32), want["row_outer"], "outer rows %d.." % r0)
    del x, out
    torch.cuda.empty_cache()


def test_cast_transpose_65536_squared():
    """fp4_cast_transpose, NVFP4 2D outer, SR, error feedback, staged, 65536 x
    65536 (2^32 elements: 8 GiB in, a 16 GiB residual, 2 GiB of codes per
    direction)."""
    R = C = 65536
    base = 999
    x = _source(R, C, 2)
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    z = torch.randn((R, C), generator=g, device="cuda", dtype=torch.float32).mul_(1e-3)
    bands = _bands(R)
    z_before = {r0: _host(z[r0:r0 + 64], np.float32).copy() for r0 in bands}
    cfg = fq.make_cfg(format="nvfp4", two_level="outer_block", outer_block_size=64, outer_2d=True,
                      rounding="stochastic", seed=78, step=6, index_base=base)
    out = fq.fp4_cast_transpose(x, cfg, residual=z)
    torch.cuda.synchronize()
    col_codes = out["col_codes"]          # [C, R / 2]
    col_scales = out["col_scales"]        # [C, R / 16]
    for r0 in bands:
        xb = _host(x[r0:r0 + 64], np.uint16)
        zo = z_before[r0].copy()
        want = ref.nv_quantize(xb, scale_fmt="e4m3", two_level="outer", obs=64, outer_2d=True, stochastic=True,
                               seed=78, step=6, index_base=base + r0 * C, residual=zo, cols=True, want_y=False)
        _same(_host(out["row_codes"][r0:r0 + 64], np.uint8), want["row_codes"], "row codes %d.." % r0)
        _same(_host(out["row_scales"][r0:r0 + 64], np.uint8), want["row_scales"], "row scales %d.." % r0)
        _same(_host(out["row_outer"].view(R // 64, C // 64)[r0 // 64], np.float32), want["row_outer"].ravel(),
              "outer band %d" % r0)
        _same(_host(col_codes[:, r0 // 2:(r0 + 64) // 2], np.uint8), want["col_codes"], "col codes %d.." % r0)
        _same(_host(col_scales[:, r0 // 16:(r0 + 64) // 16], np.uint8), want["col_scales"], "col scales %d.." % r0)
        _same(_host(z[r0:r0 + 64], np.float32), zo, "residual %d.." % r0)
    del x, z, out
    torch.cuda.empty_cache()


def test_mx_fake_quant_8_gib_of_codes_input():
    """fp4_qdq, MXFP4, 131072 x 65536 bf16 (2^33 elements, 16 GiB in and out)."""
    R, C = 131072, 65536
    x = _source(R, C, 4)
    cfg = fq.make_cfg(format="mxfp4")
    out = fq.fp4_qdq(x, cfg, with_codes=True)
    torch.cuda.synchronize()
    for r0 in _bands(R):
        xb = _host(x[r0:r0 + 64], np.uint16)
        codes, scales, y = ref.mx_qdq(xb)
        _same(_host(out["codes"][r0:r0 + 64], np.uint8), codes, "codes rows %d.." % r0)
        _same(_host(out["scales"][r0:r0 + 64], np.uint8), scales, "scales rows %d.." % r0)
        _same(_host(out["y"][r0:r0 + 64], np.uint16), y, "y rows %d.." % r0)
    del x, out
    torch.cuda.empty_cache()
