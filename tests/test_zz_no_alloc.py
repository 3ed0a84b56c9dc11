"""fp4_qdq_noalloc (the entry point for callers that cannot allocate) against
fp4_qdq with a caller workspace, through the C ABI: every output bit for bit,
on two calls in a row, the second with a smaller input, in the tensorwise mode
whose amax passes use the scratch, and in a mode that needs none."""
import ctypes as ct

import numpy as np
import pytest
import torch

import block_scaled_fp4_amax_amd as fq
from block_scaled_fp4_amax_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fq.lib()


def _outputs(R, C, with_outer):
    y = torch.empty((R, C), dtype=torch.bfloat16, device="cuda")
    y.view(torch.int16).fill_(0x5A5A)
    codes = torch.full((R, C // 2), 0xA5, dtype=torch.uint8, device="cuda")
    scales = torch.full((R, C // 16), 0xA5, dtype=torch.uint8, device="cuda")
    outer = torch.full((1,), -1.0, dtype=torch.float32, device="cuda") if with_outer else None
    return y, codes, scales, outer


def _call_noalloc(cfg, x, y, codes, scales, outer, residual):
    L = fq.lib()
    R, C = x.shape
    p = lambda t: None if t is None else ct.c_void_p(t.data_ptr())  # noqa: E731
    st = L.fp4_qdq_noalloc(ct.byref(cfg), p(x), R, C, C, p(y), p(codes), p(scales), p(outer), p(residual),
                           ct.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, fq.fp4q_status_str(st)


def _call_ws(cfg, x, y, codes, scales, outer, residual):
    L = fq.lib()
    R, C = x.shape
    nb = fq.fp4q_workspace_bytes(cfg, R, C)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
    p = lambda t: None if t is None else ct.c_void_p(t.data_ptr())  # noqa: E731
    st = L.fp4_qdq(ct.byref(cfg), p(x), R, C, C, p(y), p(codes), p(scales), p(outer), p(residual), p(ws), nb,
                   ct.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, fq.fp4q_status_str(st)


def _eq(a, b, what):
    a = a.view(torch.uint8).cpu().numpy()
    b = b.view(torch.uint8).cpu().numpy()
    bad = np.flatnonzero(a.ravel() != b.ravel())
    assert bad.size == 0, "%s: %d bytes differ, first at %d" % (what, bad.size, bad[0])


@pytest.mark.parametrize("mode", ["tensorwise", "tensorwise_sr_ef", "outer1d"])
def test_noalloc_equals_workspace_call_twice(mode):
    rng = np.random.default_rng(31)
    if mode == "outer1d":
        cfg = fq.make_cfg(format="amdfp4", two_level="outer_block", outer_block_size=64)
    elif mode == "tensorwise":
        cfg = fq.make_cfg(format="nvfp4", two_level="tensorwise")
    else:
        cfg = fq.make_cfg(format="nvfp4", two_level="tensorwise", rounding="stochastic", seed=3, step=1)
    ef = mode == "tensorwise_sr_ef"
    for R, C in ((1024, 4096), (96, 320)):        # the second call is smaller
        a = rng.standard_normal((R, C)).astype(np.float32) * np.exp(rng.standard_normal((R, 1))).astype(np.float32)
        x = torch.from_numpy(W.to_bf16(a).view(np.int16)).cuda()
        z0 = torch.from_numpy((rng.standard_normal((R, C)) * 0.01).astype(np.float32)).cuda() if ef else None
        n_outer = 1 if mode != "outer1d" else R * (C // 64)
        ya, ca, sa, _ = _outputs(R, C, False)
        oa = torch.full((n_outer,), -1.0, dtype=torch.float32, device="cuda")
        yb, cb, sb, _ = _outputs(R, C, False)
        ob = torch.full((n_outer,), -1.0, dtype=torch.float32, device="cuda")
        za = None if z0 is None else z0.clone()
        zb = None if z0 is None else z0.clone()
        _call_noalloc(cfg, x, ya, ca, sa, oa, za)
        _call_ws(cfg, x, yb, cb, sb, ob, zb)
        torch.cuda.synchronize()
        _eq(ya, yb, "%s %dx%d y" % (mode, R, C))
        _eq(ca, cb, "%s %dx%d codes" % (mode, R, C))
        _eq(sa, sb, "%s %dx%d scales" % (mode, R, C))
        _eq(oa, ob, "%s %dx%d outer" % (mode, R, C))
        if ef:
            _eq(za, zb, "%s %dx%d residual" % (mode, R, C))
