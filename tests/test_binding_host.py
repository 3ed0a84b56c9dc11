"""Host-side checks of the Python binding (no GPU, no launch): the
error-feedback state manager's bookkeeping and argument rules ("fp4-train"
README, API: ErrorFeedback), and the refusal of host tensors before any
pointer reaches the library."""
import pytest
import torch

import block_scaled_fp4_amax_amd as fq


def test_host_tensors_are_refused():
    x = torch.zeros(16, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensors"):
        fq.fp4_qdq(x, fq.make_cfg())
    with pytest.raises(ValueError, match="device tensors"):
        fq.fp4_quantize(x.float(), fq.make_cfg(format="mxfp4"))
    with pytest.raises(ValueError, match="device tensors"):
        fq.fp4_mx_project_fp8(x)


def test_error_feedback_rules():
    with pytest.raises(fq.Fp4Error):
        fq.ErrorFeedback(format="mxfp4")
    with pytest.raises(ValueError):
        fq.ErrorFeedback(fq.make_cfg(), stochastic=True)
    ef = fq.ErrorFeedback(stochastic=True, seed=7, two_level="tensorwise")
    assert ef.cfg.rounding == fq.ROUNDING["stochastic"] and ef.cfg.seed == 7
    assert ef.cfg.two_level == fq.TWO_LEVEL["tensorwise"]
    assert ef._cfg(5).step == 5 and ef.cfg.step == 0          # per-call step, stored cfg untouched
    with pytest.raises(KeyError):
        ef.residual("w")
    like = torch.zeros(32, 64, dtype=torch.bfloat16)
    r = ef.residual("w", like)
    assert r.dtype == torch.float32 and tuple(r.shape) == (32, 64) and not r.any()
    assert ef.residual("w", like) is r
    with pytest.raises(ValueError):
        ef.residual("w", torch.zeros(16, 64))
    sd = ef.state_dict()
    sd["w"] += 1
    assert not ef.residual("w").any()                          # state_dict holds copies
    ef.load_state_dict(sd)
    assert bool((ef.residual("w") == 1).all())
    with pytest.raises(ValueError):
        ef.load_state_dict({"w": torch.zeros(4, dtype=torch.float32)})
    ef.reset("w")
    with pytest.raises(KeyError):
        ef.residual("w")


def test_caller_buffers_are_size_checked_before_any_call():
    """Too-small or non-contiguous caller buffers are refused by the binding
    (the C ABI trusts its sizes); these checks run before the device check."""
    u8 = lambda *s: torch.zeros(*s, dtype=torch.uint8)  # noqa: E731
    with pytest.raises(ValueError, match="a scales"):
        fq.fp4_mm({"codes": u8(64, 64), "scales": u8(64, 3)}, {"codes": u8(32, 64), "scales": u8(32, 4)})
    with pytest.raises(ValueError, match="b codes"):
        fq.fp4_mm({"codes": u8(64, 64), "scales": u8(64, 4)}, {"codes": u8(32, 128)[:, :64], "scales": u8(32, 4)})
    with pytest.raises(ValueError, match="tiled scales|a scales"):
        fq.fp4_mm({"codes": u8(64, 64), "scales_tiled": u8(100)}, {"codes": u8(32, 64), "scales_tiled": u8(2048)})
    with pytest.raises(ValueError, match="c must be"):
        fq.fp4_mm({"codes": u8(64, 64), "scales": u8(64, 4)}, {"codes": u8(32, 64), "scales": u8(32, 4)},
                  c=torch.zeros(32, 64, dtype=torch.float32))
    with pytest.raises(ValueError, match="residual"):
        fq.fp4_qdq(torch.zeros(16, 32, dtype=torch.bfloat16), fq.make_cfg(), residual=torch.zeros(16, 16))
    with pytest.raises(ValueError, match="codes holds"):
        fq.fp4_quantize(torch.zeros(16, 32, dtype=torch.bfloat16), fq.make_cfg(), out={"codes": u8(16, 8)})
    with pytest.raises(ValueError, match="y holds"):
        fq.fp4_dequantize(u8(16, 16), u8(16, 2), None, 16, 32, fq.make_cfg(), y=torch.zeros(16, 16, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="blk_scales"):
        fq.fp4_mx_project_fp8(torch.zeros(128, 128, dtype=torch.bfloat16),
                              out={"blk_scales": torch.zeros(0, dtype=torch.float32)})
