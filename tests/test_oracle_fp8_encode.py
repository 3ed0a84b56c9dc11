"""Pins of the oracle's FP8 re-encodings of the MXFP4 projection ("MXFP4 weight
QAT recipes on MXFP8 and FP8 block-scaling hosts", Design and Correctness): the
rowwise MXFP8 encoding of the projected weight is bitwise lossless, the 128x128
block encoding is lossless within a tile's E4M3 headroom (the full payload grid
exact through a scale spread of 2^14), the columnwise 32x1 encoding is a
bounded re-quantisation.

Independent references: torch's float8_e4m3fn cast and decode (a library
implementation of the OCP E4M3FN format), the MXFP4 projection's own fixed
points, and the properties the page states."""
import numpy as np
import pytest
import torch

from block_scaled_fp4_amax_amd import workloads as W
from oracle import ref

G = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)


def e4m3_decode(b):
    """Independent decoder: torch's float8_e4m3fn view of the payload bytes."""
    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy().astype(np.float64)


def bf16_values(y):
    return (np.ascontiguousarray(y, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_e4m3_payload_equals_torch_cast():
    vals = [0.0, -0.0]
    for j in range(-20, 10):
        for g in G[1:]:
            v = g * 2.0 ** j
            if v <= 448:
                vals += [v, -v]
    rng = np.random.default_rng(0)
    vals += list(rng.uniform(0, 448, 2000)) + list(rng.uniform(0, 2.0 ** -6, 2000)) + list(-rng.uniform(0, 30, 500))
    vals += [2.0 ** -10, 3 * 2.0 ** -11, 2.0 ** -10 * 1.0000001, 447.9, 448.0]
    v32 = np.array(vals, np.float32)
    want = torch.from_numpy(v32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([ref.e4m3_payload(float(v)) for v in v32], np.uint8)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (v32[bad[:5]], got[bad[:5]], want[bad[:5]])
    # NaN: 0xFF, a NaN code of E4M3FN
    assert ref.e4m3_payload(float("nan")) == 0xFF
    assert np.isnan(e4m3_decode(np.array([0xFF], np.uint8))[0])


def _edge_weight(rows=256, cols=512):
    return W.mx_weight_8192_edges(rows=rows, cols=cols)


def test_mx8_rowwise_is_lossless_and_normalised():
    x = _edge_weight()
    o = ref.mx_project_encode(x, mx8_col=False, blk=False)
    y = bf16_values(o["y"])
    sc = o["mx8_row_scales"].astype(np.int64)
    dec = e4m3_decode(o["mx8_row"]) * np.repeat(2.0 ** (sc - 127), 32, axis=1)
    fin = np.isfinite(y)
    assert np.array_equal(dec[fin], y[fin])                        # bitwise lossless
    assert np.all(o["mx8_row"][~fin] == 0xFF) and (~fin).any()     # poisoned blocks carry NaN payloads
    # OCP normalisation: a block's largest finite magnitude sits in E4M3's top binade [256, 512)
    mag = np.abs(np.where(fin, y, 0.0)).reshape(y.shape[0], -1, 32).max(axis=2)
    top = np.abs(e4m3_decode(o["mx8_row"]) * np.isfinite(y)).reshape(y.shape[0], -1, 32).max(axis=2)
    nz = (mag > 0) & (sc > 0)
    assert nz.any() and np.all((top[nz] >= 256) & (top[nz] < 512))
    assert np.all(sc[mag == 0] == 0)


def test_mx8_rowwise_lossless_on_every_bf16_pattern():
    # every bf16 pattern as a member of a block (2048 blocks of 32)
    x = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(2048, 32)
    o = ref.mx_project_encode(x, mx8_col=False, blk=False)
    y = bf16_values(o["y"])
    dec = e4m3_decode(o["mx8_row"]) * (2.0 ** (o["mx8_row_scales"].astype(np.int64) - 127))
    fin = np.isfinite(y)
    assert np.array_equal(dec[fin], y[fin])


def test_mx8_columnwise_is_a_bounded_requantisation():
    x = _edge_weight()
    o = ref.mx_project_encode(x, mx8_row=False, blk=False)
    yt = bf16_values(o["y"]).T
    sc = np.repeat(2.0 ** (o["mx8_col_scales"].astype(np.int64) - 127), 32, axis=1)
    fin = np.isfinite(yt)
    # the payload is torch's E4M3 cast of y^T / 2^E with the stored exponent
    q = np.where(fin, yt / sc, 0.0).astype(np.float32)
    want = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = o["mx8_col"]
    assert np.array_equal(np.where(fin, got, 0), np.where(fin, want, 0))
    assert np.all(got[~fin] == 0xFF)
    # error bound: half an E4M3 step at the value's binade (step 2^-9 below 2^-6)
    dec = e4m3_decode(got) * sc
    err = np.abs(np.where(fin, dec - yt, 0.0))
    a = np.abs(np.where(fin, yt, 0.0)) / sc
    step = np.where(a >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3), 2.0 ** -9)
    assert np.all(err <= 0.5 * step * sc)
    assert (err > 0).any()            # not lossless in general: blocks mix row scales


def _spread_tile(K, spreads, rng):
    """A 128 x 128 bf16 tile of MXFP4 fixed points: every 1x32 block holds
    6 * 2^k (its own maximum) and G[m] * 2^k, with k = K - d for a spread d
    per block, so the projection reproduces the tile exactly."""
    x = np.zeros((128, 128), np.float32)
    blocks = [(i, b) for i in range(128) for b in range(4)]
    for n, (i, b) in enumerate(blocks):
        d = spreads[n % len(spreads)]
        k = K - d
        vals = np.array([6.0] + [G[1 + (t % 7)] for t in range(31)]) * 2.0 ** k
        vals *= rng.choice([-1.0, 1.0], 32)
        x[i, 32 * b:32 * b + 32] = vals
    return W.to_bf16(x)


@pytest.mark.parametrize("K", [-100, 0, 37, 120])
def test_blockwise_128_exact_through_spread_2_14(K):
    rng = np.random.default_rng(K + 1000)
    x = _spread_tile(K, list(range(0, 15)), rng)
    o = ref.mx_project_encode(x, mx8_row=False, mx8_col=False)
    y = bf16_values(o["y"])
    assert np.array_equal(y, bf16_values(x))                       # fixed points of the projection
    s = float(o["blk_scales"][0, 0])
    assert s == 2.0 ** np.round(np.log2(s))                          # a power of two
    assert 224 < 6 * 2.0 ** K / s <= 448                             # the smallest one with amax / s <= 448
    dec = e4m3_decode(o["blk"]) * s
    assert np.array_equal(dec, y)                                    # every payload exact for spreads 0..14
    assert np.array_equal(o["blk_t"], o["blk"].T)


def test_blockwise_128_loses_values_beyond_spread_2_14():
    rng = np.random.default_rng(5)
    x = _spread_tile(10, [0, 15, 16], rng)
    o = ref.mx_project_encode(x, mx8_row=False, mx8_col=False)
    y = bf16_values(o["y"])
    dec = e4m3_decode(o["blk"]) * float(o["blk_scales"][0, 0])
    assert not np.array_equal(dec, y)
    # values in E4M3's normal range (>= 2^-6 of the scale) stay exact; below it the
    # payload grid is the multiples of 2^-9 of the scale, which spreads of 15 and
    # 16 binades leave
    s = float(o["blk_scales"][0, 0])
    normal = np.abs(y) >= s * 2.0 ** -6
    assert np.array_equal(dec[normal], y[normal])
    off_grid = (~normal) & (np.abs(y) / s * 2.0 ** 9 % 1 != 0)
    assert off_grid.any() and np.all(dec[off_grid] != y[off_grid])


def test_blockwise_scale_of_an_all_zero_tile_is_one():
    x = np.zeros((128, 256), np.uint16)
    x[:, 128:] = W.to_bf16(np.full((128, 128), 3.0, np.float32))
    o = ref.mx_project_encode(x, mx8_row=False, mx8_col=False)
    assert o["blk_scales"][0, 0] == 1.0 and np.all(o["blk"][:, :128] == 0)
    assert o["blk_scales"][0, 1] == 2.0 ** np.ceil(np.log2(3.0 / 448))
