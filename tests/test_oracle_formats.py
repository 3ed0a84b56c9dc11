"""Pins for the oracle's format primitives (CPU only).

Each test checks the C oracle against something other than itself: a value
the pages print (tests/golden), a library routine (torch casts, numpy float32
division, rocRAND's Philox4x32-10), a closed form, or the exact-rational model.
"""
import ctypes as ct
import os
import subprocess
import tempfile

import numpy as np
import pytest
import torch

from oracle import exact, ref

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------- E2M1
def test_e2m1_grid_matches_printed_values(golden):
    grid = [float(r[0]) for r in golden("e2m1_grid.txt")]
    assert [ref.e2m1_value(m) for m in range(8)] == grid


def _threshold_code(a):
    """Closed form of RNE onto {0,.5,1,1.5,2,3,4,6} with ties to the even code:
    the decision points are the midpoints, and a tie goes up exactly when the
    upper neighbour has the even code (0.75 -> 1.0, 1.75 -> 2.0, 3.5 -> 4.0)."""
    a = np.asarray(a)
    if a.dtype != np.float32:
        a = a.astype(np.float64)
    f = a.dtype.type          # every decision point is exact in binary32 and binary64
    m = (a > f(0.25)).view(np.uint8).copy()
    for t, strict in ((0.75, False), (1.25, True), (1.75, False), (2.5, True), (3.5, False), (5.0, True)):
        m += (a > f(t)) if strict else (a >= f(t))
    return m


def test_e2m1_rne_midpoints_and_saturation(golden):
    limits = {r[0]: float(r[1]) for r in golden("format_limits.txt")}
    assert limits["e2m1_max"] == 6.0
    # midpoint between codes lo and lo+1: below -> lo, above -> lo+1, on it -> the even one
    mids = {0.25: 0, 0.75: 1, 1.25: 2, 1.75: 3, 2.5: 4, 3.5: 5, 5.0: 6}
    for a, lo in mids.items():
        a32 = np.float32(a)
        assert ref.e2m1_rne(float(a32)) == (lo if lo % 2 == 0 else lo + 1), a
        assert ref.e2m1_rne(float(np.nextafter(a32, np.float32(0)))) == lo, a
        assert ref.e2m1_rne(float(np.nextafter(a32, np.float32(10)))) == lo + 1, a
    for a in (6.0, 6.5, 7.0, 1e30):
        assert ref.e2m1_rne(a) == 7


def test_e2m1_rne_matches_closed_form_on_every_fp32_below_8():
    # every binary32 pattern in [0, 8) (about 1.09e9 values), in chunks
    hi = int(np.float32(8.0).view(np.uint32))
    step = 1 << 25
    for lo in range(0, hi, step):
        a = np.arange(lo, min(hi, lo + step), dtype=np.uint32).view(np.float32)
        got = ref.e2m1_rne_array(a)
        want = _threshold_code(a)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (a[bad[:4]], got[bad[:4]], want[bad[:4]])


def test_e2m1_rne_and_sr_match_exact_model():
    rng = np.random.default_rng(11)
    a = np.concatenate([rng.uniform(0, 7, 3000), np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, 6, 0])]).astype(np.float32)
    for v in a:
        assert ref.e2m1_rne(float(v)) == exact.e2m1_rne(exact.F(float(v)))
    u = rng.integers(0, 65536, a.size)
    for v, uu in zip(a, u):
        assert ref.e2m1_sr(float(v), int(uu)) == exact.e2m1_sr(exact.F(float(v)), int(uu))


def test_e2m1_sr_probability_is_ceiling_of_fraction():
    # enumerating all 2^16 draws gives P(up) = ceil(frac * 2^16) / 2^16 exactly
    for a in (np.float32(2.3), np.float32(0.1), np.float32(4.75), np.float32(1.2)):
        ups = sum(ref.e2m1_sr(float(a), u) != ref.e2m1_sr(float(a), 65535) for u in range(0, 65536, 1))
        grid = [0, .5, 1, 1.5, 2, 3, 4, 6]
        lo = max(i for i in range(8) if grid[i] <= float(a))
        frac = (float(a) - grid[lo]) / (grid[lo + 1] - grid[lo])
        assert ups == int(np.ceil(frac * 65536)), a


# ---------------------------------------------------------------- inner-scale grids
def _limits(golden):
    return {r[0]: float(r[1]) for r in golden("format_limits.txt")}


def test_scale_grid_maxima_match_printed_values(golden):
    lim = _limits(golden)
    assert ref.scale_decode("e4m3", 0x7E) == lim["e4m3_max"]
    assert ref.scale_decode("ue5m3", 0xFE) == lim["ue5m3_max"]
    assert np.isnan(ref.scale_decode("e4m3", 0x7F))
    assert np.isnan(ref.scale_decode("ue5m3", 0xFF))
    # satfinite: anything above the maximum encodes to it
    assert ref.scale_encode("e4m3", 1e6) == 0x7E
    assert ref.scale_encode("ue5m3", 1e9) == 0xFE


@pytest.mark.parametrize("fmt,top", [("e4m3", 0x7E), ("ue5m3", 0xFE)])
def test_scale_roundtrip_every_code(fmt, top):
    for c in range(top + 1):
        v = ref.scale_decode(fmt, c)
        assert ref.scale_encode(fmt, v) == c
        assert exact.scale_decode(fmt, c) == exact.F(v)


def _probe_values(lo_exp, hi_exp, grid_bits=3, stride=61, halo=128):
    """Sampled binary32 values in [2^lo_exp, 2^hi_exp): a strided sweep of every
    binade plus a halo of ulps around each 3-bit grid point and midpoint."""
    out = []
    for e in range(lo_exp, hi_exp):
        base = np.float32(2.0 ** e).view(np.uint32).astype(np.int64)
        out.append(base + np.arange(0, 1 << 23, stride))
        for k in range(2 << grid_bits):
            pt = base + (k << (23 - grid_bits - 1))
            out.append(pt + np.arange(-halo, halo + 1))
    pats = np.unique(np.concatenate(out))
    pats = pats[(pats >= 0) & (pats < 0x7F800000)]
    return pats.astype(np.uint32).view(np.float32)


def _torch_e4m3(y):
    return torch.from_numpy(np.ascontiguousarray(y, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_float8_cast():
    # every binary32 in [2^-11, 448] (every value that can round to a nonzero
    # code, and a binade below), in chunks; below 2^-11 (all of which encode to
    # zero) every 97th pattern
    lo, hi = int(np.float32(2.0 ** -11).view(np.uint32)), int(np.float32(448.0).view(np.uint32))
    step = 1 << 24
    for a in range(lo, hi + 1, step):
        y = np.arange(a, min(hi + 1, a + step), dtype=np.uint32).view(np.float32)
        got, want = ref.scale_encode_array("e4m3", y), _torch_e4m3(y)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (y[bad[:4]], got[bad[:4]], want[bad[:4]])
    tiny = np.arange(0, lo, 97, dtype=np.uint32).view(np.float32)
    np.testing.assert_array_equal(ref.scale_encode_array("e4m3", tiny), _torch_e4m3(tiny))
    assert not ref.scale_encode_array("e4m3", tiny).any()


def test_ue5m3_encode_pinned_to_e4m3_by_exponent_shift():
    """UE5M3 code c equals E4M3 code c divided by 2^8 for c <= 0x7E (bias 15 vs
    7, same 3-bit mantissa), and its normal range is self-similar under 2^8, so
    torch's E4M3 cast pins UE5M3 over its whole range."""
    # low range: codes identical after scaling by 2^8
    y = _probe_values(-22, 1)
    y = y[y <= 1.75]
    np.testing.assert_array_equal(ref.scale_encode_array("ue5m3", y), _torch_e4m3(y * np.float32(256.0)))
    # high range [448, 114688]: value(y) = 2^8 * value(y / 2^8)
    y2 = _probe_values(9, 17)
    y2 = y2[(y2 >= 448.0) & (y2 <= 114688.0)]
    got = np.array([ref.scale_decode("ue5m3", c) for c in ref.scale_encode_array("ue5m3", y2)])
    e4 = _torch_e4m3(y2 / np.float32(256.0))
    want = np.array([ref.scale_decode("e4m3", c) for c in e4]) * 256.0
    np.testing.assert_array_equal(got, want)
    assert ref.scale_encode("ue5m3", 114688.0 * 1.2) == 0xFE


def test_ue8m0_decode_rules(golden):
    lim = _limits(golden)
    assert ref.ue8m0_decode(0) == 2.0 ** lim["ue8m0_code0_log2"]
    assert np.isnan(ref.ue8m0_decode(int(lim["ue8m0_nan_code"])))
    assert ref.ue8m0_decode(127) == 1.0
    assert ref.ue8m0_decode(254) == 2.0 ** 127


# ---------------------------------------------------------------- bf16 / fp32
def test_bf16_cast_matches_torch():
    rng = np.random.default_rng(5)
    f = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(1e3),
        (rng.integers(0, 0x7F800000, 200000, dtype=np.uint32)).view(np.float32),
        (np.float32([1.0, 3.0]).view(np.uint32)[:, None] + np.arange(0x7FF0, 0x8011)).ravel().astype(np.uint32).view(np.float32),
        np.float32([0.0, -0.0, 2.0 ** -149, 2.0 ** -133, 3.3895e38, -1.0]),
    ])
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ref.f32_to_bf16(f), want)
    assert ref.f32_to_bf16(np.float32([np.nan]))[0] == 0x7FC0


def test_fp32_division_matches_numpy():
    rng = np.random.default_rng(6)
    a = rng.integers(0, 0x7F000000, 300000, dtype=np.uint32).view(np.float32)
    b = rng.integers(1, 0x7F000000, 300000, dtype=np.uint32).view(np.float32)
    with np.errstate(all="ignore"):
        want = a / b
    np.testing.assert_array_equal(ref.div_f32(a, b).view(np.uint32), want.view(np.uint32))


# ---------------------------------------------------------------- Philox4x32-10
@pytest.fixture(scope="module")
def rocrand_pin():
    src = os.path.join(os.path.dirname(__file__), "pins", "rocrand_philox.cpp")
    d = tempfile.mkdtemp(prefix="fp4pin")
    so = os.path.join(d, "libpin.so")
    try:
        subprocess.run(["g++", "-O1", "-std=c++17", "-shared", "-fPIC", "-I/opt/rocm/include",
                        "-D__HIP_PLATFORM_AMD__", src, "-o", so], check=True, capture_output=True)
    except (OSError, subprocess.CalledProcessError) as e:  # pragma: no cover
        pytest.skip("rocRAND host header not usable: %s" % e)
    L = ct.CDLL(so)
    L.pin_philox.restype = None
    L.pin_philox.argtypes = [ct.c_uint64, ct.c_uint64, ct.c_uint64, ct.c_void_p]
    return L


def _pin(L, seed, step, c):
    out = np.zeros(4, np.uint32)
    L.pin_philox(seed, step, c, out.ctypes.data_as(ct.c_void_p))
    return out


def test_philox_matches_rocrand(rocrand_pin):
    rng = np.random.default_rng(7)
    cases = [(0, 0, 0), (7, 3, 1), (5, 2, 123456), (2 ** 64 - 1, 2 ** 64 - 1, 2 ** 61 - 1)]
    # rocRAND positions the counter through a 64-bit element offset 4*c, so the
    # pin covers block counters c < 2^62 (element indices < 2^65)
    cases += [(int(rng.integers(0, 2 ** 63)), int(rng.integers(0, 2 ** 63)), int(rng.integers(0, 2 ** 62)))
              for _ in range(300)]
    for seed, step, c in cases:
        ctr = [c & 0xFFFFFFFF, c >> 32, step & 0xFFFFFFFF, step >> 32]
        key = [seed & 0xFFFFFFFF, seed >> 32]
        np.testing.assert_array_equal(ref.philox4x32_10(ctr, key), _pin(rocrand_pin, seed, step, c))


def test_sr_u16_lane_mapping(rocrand_pin):
    for seed, step, c in [(7, 3, 0), (7, 3, 99), (5, 1, 2 ** 40 + 5)]:
        words = _pin(rocrand_pin, seed, step, c)
        for lane in range(8):
            want = (int(words[lane >> 1]) >> (16 * (lane & 1))) & 0xFFFF
            assert ref.sr_u16(seed, step, 8 * c + lane) == want


def test_sr_u16_uniformity():
    u = ref.sr_u16_array(7, 3, 0, 1 << 20)
    for part in (u >> 8, u & 0xFF):
        counts = np.bincount(part, minlength=256)
        exp = u.size / 256
        chi2 = ((counts - exp) ** 2 / exp).sum()
        assert chi2 < 400, chi2          # 255 dof: mean 255, sd ~22.6
    assert abs(u.mean() - 32767.5) < 200
