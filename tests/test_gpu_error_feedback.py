"""GPU parity of the error-feedback state manager ("fp4-train" README, API:
ErrorFeedback, and the usage it shows: W = ef.qdq(name, W - lr * grad,
step=step)) against the oracle run step by step with its own residual, bit for
bit: dequantised weights and residuals after every step, bf16 and FP32
weights, RNE and stochastic rounding, and a state_dict round trip.

The weight chain is computed on the host from the oracle's outputs
(x_{t+1} = y_t - lr * g_t with seeded g_t) and handed to both sides."""
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


def host_bits(t):
    torch.cuda.synchronize()
    a = t.detach().cpu().contiguous()
    if a.dtype == torch.bfloat16:
        return a.view(torch.int16).numpy().view(np.uint16)
    return a.numpy().view(np.uint32)


def oracle_bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


def to_dev(x):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(x).cuda()


def next_weight(y, t, lr=np.float32(0.01)):
    """x_{t+1} = y_t - lr * g_t in binary32, rounded back to the weight's dtype."""
    g = np.random.default_rng(900 + t).standard_normal(y.shape).astype(np.float32)
    if y.dtype == np.uint16:
        return W.to_bf16(W.from_bf16(y) - lr * g)
    return (y - lr * g).astype(np.float32)


CASES = [
    # fmt, scale_fmt (oracle), two_level, obs, sr, dtype
    ("nvfp4", "e4m3", "none", 0, False, "bf16"),
    ("nvfp4", "e4m3", "tensorwise", 0, True, "bf16"),
    ("amdfp4", "ue5m3", "outer", 64, True, "bf16"),
    ("nvfp4", "e4m3", "outer", 32, True, "fp32"),
    ("nvfp4", "e4m3", "none", 0, False, "fp32"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(str(v) for v in c))
def test_error_feedback_steps_match_the_oracle(case):
    fmt, osf, tl, obs, sr, dtype = case
    R, C = 96, 320
    x = W.fp32_weights(77, R, C)
    x = W.to_bf16(x) if dtype == "bf16" else x
    gtl = {"none": "none", "tensorwise": "tensorwise", "outer": "outer_block"}[tl]
    ef = fq.ErrorFeedback(format=fmt, two_level=gtl, outer_block_size=obs, stochastic=sr, seed=21)
    res = np.zeros((R, C), np.float32)
    for t in range(4):
        want = ref.nv_quantize(x, scale_fmt=osf, two_level=tl, obs=obs, stochastic=sr, seed=21, step=t,
                               residual=res, y_dtype=dtype)
        y = ef.qdq("layer0.weight", to_dev(x), step=t)
        np.testing.assert_array_equal(host_bits(y), oracle_bits(want["row_y"]), err_msg="step %d y" % t)
        np.testing.assert_array_equal(host_bits(ef.residual("layer0.weight")), res.view(np.uint32),
                                      err_msg="step %d residual" % t)
        x = next_weight(want["row_y"], t)


def test_state_dict_round_trip_continues_the_same_chain():
    R, C = 64, 256
    x0 = W.to_bf16(W.fp32_weights(5, R, C))
    kw = dict(format="nvfp4", two_level="tensorwise", stochastic=True, seed=4)
    a = fq.ErrorFeedback(**kw)
    b = fq.ErrorFeedback(**kw)
    xs = [x0]
    res = np.zeros((R, C), np.float32)
    for t in range(4):
        want = ref.nv_quantize(xs[-1], two_level="tensorwise", stochastic=True, seed=4, step=t, residual=res)
        xs.append(next_weight(want["row_y"], t))
    ya = [a.qdq("w", to_dev(xs[t]), step=t) for t in range(4)]
    for t in range(2):
        b.qdq("w", to_dev(xs[t]), step=t)
    c = fq.ErrorFeedback(**kw)
    c.load_state_dict(b.state_dict())
    yc = [c.qdq("w", to_dev(xs[t]), step=t) for t in (2, 3)]
    for t, y in zip((2, 3), yc):
        np.testing.assert_array_equal(host_bits(y), host_bits(ya[t]), err_msg="step %d after reload" % t)
    np.testing.assert_array_equal(host_bits(c.residual("w")), host_bits(a.residual("w")))
    np.testing.assert_array_equal(host_bits(a.residual("w")), res.view(np.uint32))


def test_quantize_updates_the_same_residual():
    R, C = 32, 128
    x = W.to_bf16(W.fp32_weights(9, R, C))
    ef = fq.ErrorFeedback(format="nvfp4")
    res = np.zeros((R, C), np.float32)
    want = ref.nv_quantize(x, residual=res)
    q = ef.quantize("w", to_dev(x))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q["codes"].cpu().numpy(), want["row_codes"])
    np.testing.assert_array_equal(q["scales"].cpu().numpy(), want["row_scales"])
    np.testing.assert_array_equal(host_bits(ef.residual("w")), res.view(np.uint32))
