"""Checkpoint and resume of the grouped error-feedback chain.

The only state carried between calls is the caller's FP32 residual and the
(seed, step) of the counter-based generator ("fp4-train" README, API: the
residual is updated in place; Method: error feedback with stochastic
rounding).  Resuming at step 2 from a residual saved after step 1 must
therefore give, bit for bit, the outputs and the residual of an uninterrupted
run.  Both runs go through the library, so this checks the resume contract (no
hidden state in the library, steps independent of launch history), not the
arithmetic, which the oracle tests cover."""
import io

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


def _host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().contiguous().numpy().view(np.uint8)


def _steps(rows, cfg_kw, residual, steps, staged):
    outs = []
    for t, w in steps:
        g = fq.make_cfg(step=t, **cfg_kw)
        out = fq.fp4_cast_transpose_grouped(torch.from_numpy(w.view(np.int16)).cuda(), rows, g, residual=residual,
                                            staged=staged)
        outs.append({k: _host(v) for k, v in out.items() if v is not None})
    return outs


@pytest.mark.parametrize("size,staged", [("32x2880", True), ("6x192", False), ("6x192", True)])
def test_grouped_chain_resumes_bit_for_bit_from_a_saved_residual(size, staged):
    if size == "32x2880":
        E, R, C = 32, 2880, 2880
    else:
        E, R, C = 6, 192, 192
    rows = [R] * E
    w = W.experts_32x2880(experts=E, rows=R, cols=C)
    ws = [w]
    for t in range(3):
        ws.append(W.apply_expert_update(ws[-1], W.expert_update(t, w.shape)))
    cfg_kw = dict(format="nvfp4", two_level="outer_block", outer_block_size=64, outer_2d=True, rounding="stochastic",
                  seed=5)
    # uninterrupted: steps 0..3
    za = torch.zeros((E * R, C), dtype=torch.float32, device="cuda")
    straight = _steps(rows, cfg_kw, za, [(t, ws[t]) for t in range(4)], staged)
    # steps 0..1, checkpoint the residual through host memory, new device buffer, steps 2..3
    zb = torch.zeros((E * R, C), dtype=torch.float32, device="cuda")
    _steps(rows, cfg_kw, zb, [(t, ws[t]) for t in range(2)], staged)
    buf = io.BytesIO()
    np.save(buf, zb.cpu().numpy())
    del zb
    torch.cuda.empty_cache()
    buf.seek(0)
    zc = torch.from_numpy(np.load(buf)).cuda()
    resumed = _steps(rows, cfg_kw, zc, [(t, ws[t]) for t in (2, 3)], staged)
    for t, (a, b) in zip((2, 3), zip(straight[2:], resumed)):
        for k in a:
            np.testing.assert_array_equal(a[k], b[k], err_msg="step %d %s after resume" % (t, k))
    np.testing.assert_array_equal(_host(za), _host(zc), err_msg="final residual after resume")
