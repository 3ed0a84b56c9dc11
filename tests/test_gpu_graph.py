"""Entry points captured in a HIP graph replay what they compute eagerly.

Each case runs once eagerly, once more on a side stream (so that every launch
path has run before capture), is captured with torch.cuda.graph, and is then
replayed three times.  Before each replay its mutable inputs (the residual)
are restored and its outputs are overwritten with a fill kernel; between
replays the program runs unrelated eager work and synchronises.  Every replay
must equal the eager outputs byte for byte.  The cases cover the staged
grouped step with its gather, direct stores, the multi-launch tensorwise path
with its workspace, the one-launch tensorwise path, the FP8 re-encode, the
rowwise kernel with a residual and the allocation-free entry point."""
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


def _bf16(R, C, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    a = (rng.standard_normal((R, C)) * scale).astype(np.float32)
    a *= np.exp(rng.standard_normal((R, 1))).astype(np.float32)
    return torch.from_numpy(W.to_bf16(a).view(np.int16)).cuda()


def _tensors(out):
    return {k: v for k, v in out.items() if isinstance(v, torch.Tensor)}


def _snapshot(ts):
    torch.cuda.synchronize()
    return {k: v.detach().cpu().clone() for k, v in ts.items()}


def _scramble(ts):
    """Overwrite the outputs (not the residual: it is read as well as written,
    and is restored before each replay instead)."""
    for k, v in ts.items():
        if k == "residual":
            continue
        if v.dtype in (torch.float32, torch.bfloat16):
            v.fill_(float("nan"))
        else:
            v.fill_(0x5A)


def _other_work():
    y = fq.fp4_qdq(_bf16(128, 256, 99), fq.make_cfg(format="mxfp4"))["y"]
    torch.cuda.synchronize()
    return y


def _replays_equal_eager(run, reset):
    reset()
    eager = _snapshot(_tensors(run()))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        reset()
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = _tensors(run())
    assert set(outs) == set(eager)
    for rep in range(3):
        reset()
        _scramble(outs)
        torch.cuda.synchronize()
        g.replay()
        got = _snapshot(outs)
        for k in eager:
            a, b = eager[k].contiguous().view(torch.uint8).numpy(), got[k].contiguous().view(torch.uint8).numpy()
            bad = np.flatnonzero(a.ravel() != b.ravel())
            assert bad.size == 0, "replay %d, %s: %d bytes differ from the eager call" % (rep, k, bad.size)
        _other_work()


def _residual(R, C, seed):
    z0 = torch.from_numpy((np.random.default_rng(seed).standard_normal((R, C)) * 0.01).astype(np.float32)).cuda()
    z = z0.clone()
    return z, lambda: z.copy_(z0)


def test_grouped_staged_sr_ef():
    rows = [192, 64, 128]
    C = 320
    x = _bf16(sum(rows), C, 1)
    z, reset = _residual(sum(rows), C, 2)
    cfg = fq.make_cfg(format="nvfp4", two_level="outer_block", outer_block_size=64, outer_2d=True,
                      rounding="stochastic", seed=3, step=4)

    def run():
        out = fq.fp4_cast_transpose_grouped(x, rows, cfg, residual=z)
        out["residual"] = z
        return out
    _replays_equal_eager(run, reset)


def test_cast_transpose_direct_1d_sr():
    x = _bf16(128, 256, 5)
    cfg = fq.make_cfg(format="amdfp4", two_level="outer_block", outer_block_size=64, rounding="stochastic",
                      seed=6, step=7)
    _replays_equal_eager(lambda: fq.fp4_cast_transpose(x, cfg, staged=False), lambda: None)


@pytest.mark.parametrize("R,C", [(1024, 1024), (256, 256)], ids=["two-pass", "one-launch"])
def test_tensorwise_sr_qdq(R, C):
    x = _bf16(R, C, 8)
    cfg = fq.make_cfg(format="nvfp4", two_level="tensorwise", rounding="stochastic", seed=9, step=1)
    _replays_equal_eager(lambda: fq.fp4_qdq(x, cfg, with_codes=True), lambda: None)


def test_rowwise_1d_with_residual():
    x = _bf16(96, 512, 10)
    z, reset = _residual(96, 512, 11)
    cfg = fq.make_cfg(format="nvfp4", two_level="outer_block", outer_block_size=32, rounding="stochastic",
                      seed=12, step=2)

    def run():
        out = fq.fp4_quantize(x, cfg, residual=z)
        out["residual"] = z
        return out
    _replays_equal_eager(run, reset)


def test_mx_project_fp8():
    x = _bf16(256, 384, 13, scale=0.02)
    _replays_equal_eager(lambda: fq.fp4_mx_project_fp8(x), lambda: None)


def test_qdq_noalloc_tensorwise():
    R, C = 1024, 768
    x = _bf16(R, C, 14)
    cfg = fq.make_cfg(format="nvfp4", two_level="tensorwise", rounding="stochastic", seed=15, step=3)
    y = torch.empty((R, C), dtype=torch.bfloat16, device="cuda")
    codes = torch.empty((R, C // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((R, C // 16), dtype=torch.uint8, device="cuda")
    outer = torch.empty(1, dtype=torch.float32, device="cuda")
    _replays_equal_eager(lambda: fq.fp4_qdq_noalloc(x, cfg, y=y, codes=codes, scales=scales, outer=outer),
                         lambda: None)
