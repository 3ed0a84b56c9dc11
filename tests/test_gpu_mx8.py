"""GPU parity of the MXFP4 projection with its FP8 re-encodings ("MXFP4 weight
QAT recipes on MXFP8 and FP8 block-scaling hosts", Design and Correctness)
against the CPU oracle, bit for bit, through the C ABI: the bf16 projection,
MXFP8 rowwise and columnwise payloads and UE8M0 scales, the 128x128 payload,
its transpose and the FP32 block scales.  Inputs are seeded and synthetic,
including the MXFP4 edge injections (+-0, subnormals, inf / NaN poisoning,
the scale cap) and tiles of tiny values whose block scale lies below 2^-127.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp4_amax_amd as fq
from block_scaled_fp4_amax_amd import workloads as W
from oracle import ref

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

KEYS = ("y", "mx8_row", "mx8_row_scales", "mx8_col", "mx8_col_scales", "blk", "blk_t", "blk_scales")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fq.lib()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def host(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.cpu().numpy().view(np.uint32)
    return t.cpu().numpy()


def want_bits(k, v):
    return v.view(np.uint32) if k == "blk_scales" else v


def same(gpu, want, what):
    gpu = np.asarray(gpu).reshape(want.shape)
    bad = np.flatnonzero(gpu.ravel() != want.ravel())
    assert bad.size == 0, "%s: %d of %d differ; first at flat %d: gpu %s oracle %s" % (
        what, bad.size, want.size, bad[0], hex(int(gpu.ravel()[bad[0]])), hex(int(want.ravel()[bad[0]])))


def prefilled(x, **flags):
    """Outputs pre-filled with 0xA5 so unwritten bytes fail the comparison."""
    R, C = x.shape
    shapes = {"y": ((R, C), torch.bfloat16), "mx8_row": ((R, C), torch.uint8), "mx8_row_scales": ((R, C // 32), torch.uint8),
              "mx8_col": ((C, R), torch.uint8), "mx8_col_scales": ((C, R // 32), torch.uint8),
              "blk": ((R, C), torch.uint8), "blk_t": ((C, R), torch.uint8),
              "blk_scales": ((R // 128, C // 128), torch.float32)}
    group = {"y": "y", "mx8_row": "mx8_row", "mx8_row_scales": "mx8_row", "mx8_col": "mx8_col",
             "mx8_col_scales": "mx8_col", "blk": "blk", "blk_t": "blk", "blk_scales": "blk"}
    out = {}
    for k, (shp, dt) in shapes.items():
        if flags.get(group[k], True):
            t = torch.empty(shp, dtype=dt, device="cuda")
            t.view(torch.uint8).fill_(0xA5)
            out[k] = t
    return out


def check_all(x, what, **flags):
    want = ref.mx_project_encode(x, **flags)
    out = fq.fp4_mx_project_fp8(dev(x), out=prefilled(x, **flags), **flags)
    for k in KEYS:
        if k in want:
            same(host(out[k]), want_bits(k, want[k]), "%s %s" % (what, k))
    return out


def test_edge_weight_every_output():
    x = W.mx_weight_8192_edges(rows=512, cols=1024)
    check_all(x, "edges 512x1024")


def test_every_bf16_pattern():
    x = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(512, 128)
    check_all(x, "all bf16 patterns")
    check_all(np.ascontiguousarray(x.reshape(128, 512)), "all bf16 patterns 128x512")


def test_ragged_shape_without_128_blocks():
    rng = np.random.default_rng(3)
    x = W.to_bf16(rng.standard_normal((96, 160)).astype(np.float32) * np.float32(0.02))
    check_all(x, "96x160", blk=False)
    check_all(np.ascontiguousarray(x[:, :96]), "96x96 rows only", blk=False, mx8_col=False)


def test_strided_source():
    full = W.mx_weight_8192_edges(rows=256, cols=512)
    x = np.ascontiguousarray(full[:, :384])
    want = ref.mx_project_encode(x)
    out = fq.fp4_mx_project_fp8(dev(full)[:, :384])
    for k in KEYS:
        same(host(out[k]), want_bits(k, want[k]), "strided " + k)


def test_tiles_of_tiny_values():
    # tile (0, 0): largest value 1.875 * 2^-120, projected to 6 * 2^-121, scale 2^-127;
    # tile (1, 2): largest value 2^-127, scale 2^-135 (below the scaled conversion's range);
    # tile (1, 1): all zero, scale 1
    rng = np.random.default_rng(4)
    x = W.to_bf16(rng.standard_normal((256, 384)).astype(np.float32) * np.float32(0.02))
    tiny = np.array([0x0000, 0x8000, 0x0001, 0x8003, 0x0040, 0x0020, 0x00C0, 0x0100, 0x0080, 0x03F0], np.uint16)
    x[:128, :128] = rng.choice(tiny, size=(128, 128))
    x[128:, 256:] = rng.choice(tiny[:6], size=(128, 128))
    x[128:, 128:256] = 0
    out = check_all(x, "tiny tiles")
    s = host(out["blk_scales"]).view(np.float32)
    assert s[0, 0] == 2.0 ** -127 and s[1, 2] == 2.0 ** -135 and s[1, 1] == 1.0


def test_output_subsets_equal_the_full_call():
    x = W.mx_weight_8192_edges(rows=256, cols=256)
    full = fq.fp4_mx_project_fp8(dev(x))
    for flags in ({"y": False, "mx8_col": False, "blk": False}, {"y": False, "mx8_row": False, "blk": False},
                  {"y": False, "mx8_row": False, "mx8_col": False}, {"mx8_row": False, "mx8_col": False, "blk": False}):
        part = fq.fp4_mx_project_fp8(dev(x), **flags)
        for k, v in part.items():
            same(host(v), host(full[k]), "subset %s %s" % (sorted(flags), k))


def test_weight_8192_full_size_row_bands():
    """The 8192 x 8192 edge-injected weight with every output, checked on all
    64 128-row bands against the oracle run on each band (every output of a
    band depends on that band only)."""
    x = W.mx_weight_8192_edges()
    out = fq.fp4_mx_project_fp8(dev(x))
    R = C = 8192
    for b in range(R // 128):
        rows = slice(128 * b, 128 * b + 128)
        want = ref.mx_project_encode(np.ascontiguousarray(x[rows]))
        same(host(out["y"][rows]), want["y"], "band %d y" % b)
        same(host(out["mx8_row"][rows]), want["mx8_row"], "band %d mx8_row" % b)
        same(host(out["mx8_row_scales"][rows]), want["mx8_row_scales"], "band %d mx8_row_scales" % b)
        same(host(out["mx8_col"][:, rows]), want["mx8_col"], "band %d mx8_col" % b)
        same(host(out["mx8_col_scales"][:, 4 * b:4 * b + 4]), want["mx8_col_scales"], "band %d mx8_col_scales" % b)
        same(host(out["blk"][rows]), want["blk"], "band %d blk" % b)
        same(host(out["blk_t"][:, rows]), want["blk_t"], "band %d blk_t" % b)
        same(host(out["blk_scales"][b:b + 1]), want["blk_scales"].view(np.uint32), "band %d blk_scales" % b)
