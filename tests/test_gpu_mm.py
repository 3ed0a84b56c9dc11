"""GPU parity of the FP4 GEMM consumer fp4_mm (C = A . B^T with MXFP4
operands, "fp4-train" README, API: fp4_mm; Correctness: equal to the
dequantise-then-multiply path) against the oracle's binary64 GEMM.

Products are exact; the binary32 accumulation order is the kernel's, so the
bar is |C - c| <= (K - 1) 2^-24 s with s = sum_k |a_ik b_jk| from the oracle
(the standard bound for any summation order), and bit-exact where every
partial sum is a binary32 number (operand scales within 2^-1 .. 2^1 and
K <= 1024: all sums are multiples of 2^-4 below 2^18)."""
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


def operand(rng, rows, K, lo, hi):
    return (rng.integers(0, 256, (rows, K // 2), dtype=np.uint8), rng.integers(lo, hi, (rows, K // 32), dtype=np.uint8))


def dev_operand(x, layout, check_tiled=False):
    """{"codes", "scales"} (rowwise scales) or {"codes", "scales_tiled"} (the
    GEMM-ready layout, converted on the device and, when asked, compared with
    the oracle's definition of the layout)."""
    d = lambda v: torch.from_numpy(np.ascontiguousarray(v)).cuda()  # noqa: E731
    codes, scales = x
    if layout == "row":
        return {"codes": d(codes), "scales": d(scales)}
    K = codes.shape[1] * 2
    tiled = fq.fp4_mx_scales_tiled(d(scales), K)
    if check_tiled:
        torch.cuda.synchronize()
        np.testing.assert_array_equal(tiled.cpu().numpy(), ref.mx_scales_tiled(scales, scales.shape[0], K))
    return {"codes": d(codes), "scales_tiled": tiled}


def gpu_mm(a, b, dtype=torch.float32, layout="row"):
    small = a[0].size + b[0].size < (1 << 22)
    out = fq.fp4_mm(dev_operand(a, layout, small), dev_operand(b, layout, small), out_dtype=dtype)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def within_bound(got, c, s, K, what, bf16=False):
    bound = (K - 1) * 2.0 ** -24 * s + 2.0 ** -140
    if bf16:
        bound = bound + 2.0 ** -8 * np.abs(c)
    bad = np.flatnonzero(~(np.abs(got - c) <= bound))
    assert bad.size == 0, "%s: %d of %d outside the bound; first flat %d: gpu %r oracle %r bound %r" % (
        what, bad.size, c.size, bad[0], got.ravel()[bad[0]], c.ravel()[bad[0]], bound.ravel()[bad[0]])


@pytest.mark.parametrize("layout", ["row", "tiled"])
@pytest.mark.parametrize("M,N,K", [(300, 290, 1024), (256, 256, 64), (1, 515, 960), (37, 1, 128)])
def test_exact_when_every_partial_sum_is_representable(M, N, K, layout):
    rng = np.random.default_rng(M * 7 + N + K)
    a, b = operand(rng, M, K, 126, 129), operand(rng, N, K, 126, 129)
    c, _ = ref.mx_mm(*a, *b, M, N, K)
    got = gpu_mm(a, b, layout=layout)
    np.testing.assert_array_equal(got, c)


@pytest.mark.parametrize("layout", ["row", "tiled"])
@pytest.mark.parametrize("M,N,K", [(333, 517, 2880), (512, 512, 512), (64, 768, 4096), (700, 90, 192)])
def test_within_the_accumulation_bound(M, N, K, layout):
    rng = np.random.default_rng(M + N * 3 + K)
    a, b = operand(rng, M, K, 100, 150), operand(rng, N, K, 100, 150)
    c, s = ref.mx_mm(*a, *b, M, N, K)
    within_bound(gpu_mm(a, b, layout=layout), c, s, K, "fp32 C")
    within_bound(gpu_mm(a, b, torch.bfloat16, layout=layout), c, s, K, "bf16 C", bf16=True)


def test_strided_output_and_untouched_padding():
    rng = np.random.default_rng(9)
    M, N, K = 130, 200, 256
    a, b = operand(rng, M, K, 120, 135), operand(rng, N, K, 120, 135)
    c, s = ref.mx_mm(*a, *b, M, N, K)
    d = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()  # noqa: E731
    full = torch.full((M, 232), -7.0, dtype=torch.float32, device="cuda")
    fq.fp4_mm({"codes": d(a[0]), "scales": d(a[1])}, {"codes": d(b[0]), "scales": d(b[1])}, c=full[:, :N])
    torch.cuda.synchronize()
    f = full.cpu().numpy().astype(np.float64)
    within_bound(f[:, :N], c, s, K, "strided C")
    assert np.all(f[:, N:] == -7.0)


def test_quantise_then_multiply_tensors():
    """fp4_mm on bf16 / fp32 tensors quantises them (MXFP4) first: the result
    is the product of the oracle's quantised operands."""
    rng = np.random.default_rng(11)
    M, N, K = 257, 300, 2880
    xa = W.to_bf16(rng.standard_normal((M, K)).astype(np.float32))
    xb = rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02)
    ac, asc, _ = ref.mx_qdq(xa)
    bc, bsc, _ = ref.mx_qdq(xb)
    c, s = ref.mx_mm(ac, asc, bc, bsc, M, N, K)
    ta = torch.from_numpy(xa.view(np.int16)).cuda().view(torch.bfloat16)
    tb = torch.from_numpy(xb).cuda()
    got = fq.fp4_mm(ta, tb, out_dtype=torch.float32)
    torch.cuda.synchronize()
    within_bound(got.cpu().numpy().astype(np.float64), c, s, K, "quantise-then-multiply")


def test_k_zero_writes_zeros():
    d = torch.full((5, 7), 3.0, dtype=torch.float32, device="cuda")
    z = torch.empty((5, 0), dtype=torch.uint8, device="cuda")
    e = torch.empty((7, 0), dtype=torch.uint8, device="cuda")
    fq.fp4_mm({"codes": z, "scales": z}, {"codes": e, "scales": e}, c=d)
    torch.cuda.synchronize()
    assert bool((d == 0).all())


@pytest.mark.parametrize("layout", ["row", "tiled"])
def test_gemm_8192_sampled_rows(layout):
    """The 8192 x 8192 x 8192 GEMM at full size; 48 sampled rows of C (rows
    are independent) against the oracle."""
    rng = np.random.default_rng(12)
    M = N = K = 8192
    a, b = operand(rng, M, K, 115, 135), operand(rng, N, K, 115, 135)
    got = gpu_mm(a, b, layout=layout)
    rows = np.sort(rng.choice(M, 48, replace=False))
    rows[0], rows[-1] = 0, M - 1
    c, s = ref.mx_mm(a[0][rows], a[1][rows], *b, len(rows), N, K)
    within_bound(got[rows], c, s, K, "8192^3 sampled rows")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("ldc", [520, 517])
def test_whole_tiles_into_padded_c(dtype, ldc):
    """512 x 512 (whole 256 x 256 tiles) into C with row pitch ldc: 16-byte
    aligned rows take the staged 16-byte stores, odd pitches the per-element
    stores; the padding columns stay untouched."""
    rng = np.random.default_rng(ldc)
    M, N, K = 512, 512, 384
    a, b = operand(rng, M, K, 120, 135), operand(rng, N, K, 120, 135)
    c, s = ref.mx_mm(*a, *b, M, N, K)
    full = torch.full((M, ldc), -7.0, dtype=dtype, device="cuda")
    fq.fp4_mm(dev_operand(a, "tiled"), dev_operand(b, "tiled"), c=full[:, :N])
    torch.cuda.synchronize()
    f = full.float().cpu().numpy().astype(np.float64)
    within_bound(f[:, :N], c, s, K, "C ldc=%d" % ldc, bf16=dtype == torch.bfloat16)
    assert np.all(f[:, N:] == -7.0)


@pytest.mark.parametrize("M,N,K", [(512, 768, 512), (8192, 8192, 8192)])
def test_graph_replays_equal_eager(M, N, K):
    """fp4_mm captured in a HIP graph (after one eager call of the variant):
    three replays, with eager launches in between, each equal to the eager C
    (the second shape takes the direct-to-LDS kernel)."""
    rng = np.random.default_rng(21)
    a, b = operand(rng, M, K, 120, 135), operand(rng, N, K, 120, 135)
    A, B = dev_operand(a, "tiled"), dev_operand(b, "tiled")
    eager = fq.fp4_mm(A, B, out_dtype=torch.float32)
    torch.cuda.synchronize()
    want = eager.cpu().numpy().view(np.uint32).copy()
    c = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fq.fp4_mm(A, B, c=c)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fq.fp4_mm(A, B, c=c)
    for rep in range(3):
        c.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(c.cpu().numpy().view(np.uint32), want, err_msg="replay %d" % rep)
        fq.fp4_mm(B, A, out_dtype=torch.float32)          # unrelated eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("M,N,K,dtype", [(8192, 8192, 8192, torch.bfloat16), (8192, 8192, 8192, torch.float32),
                                         (8100, 8200, 8256, torch.float32), (8192, 8192, 16384, torch.bfloat16),
                                         (300, 290, 1024, torch.float32), (333, 517, 2880, torch.bfloat16),
                                         (1, 515, 960, torch.float32), (700, 90, 768, torch.float32),
                                         (257, 1000, 4096, torch.bfloat16), (2048, 1, 1600, torch.float32)])
def test_direct_lds_kernel_equals_register_staged(M, N, K, dtype):
    """With GEMM-ready scales and K of at least three 256-value K-tiles the
    library takes the direct-to-LDS kernel (only four of its eight waves load);
    with rowwise scales the register-staged one.  Both issue the same
    instructions in the same K order, so C must agree bit for bit over the
    whole matrix, ragged edges (partial tiles, single rows and columns, K tails)
    included; sampled rows of the direct kernel's C are checked against the
    oracle as well."""
    rng = np.random.default_rng(M + N + K)
    a, b = operand(rng, M, K, 115, 135), operand(rng, N, K, 115, 135)
    A_row, B_row = dev_operand(a, "row"), dev_operand(b, "row")
    A_til, B_til = dev_operand(a, "tiled"), dev_operand(b, "tiled")
    staged = fq.fp4_mm(A_row, B_row, out_dtype=dtype)
    direct = fq.fp4_mm(A_til, B_til, out_dtype=dtype)
    torch.cuda.synchronize()
    bits = torch.int16 if dtype == torch.bfloat16 else torch.int32
    same = staged.view(bits) == direct.view(bits)
    assert bool(same.all()), "%d of %d elements differ" % (int((~same).sum()), same.numel())
    rows = np.unique(np.clip([0, 1, 255, 256, M // 2, M - 2, M - 1], 0, M - 1))
    c, s = ref.mx_mm(a[0][rows], a[1][rows], *b, len(rows), N, K)
    got = direct[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    within_bound(got, c, s, K, "direct-to-LDS sampled rows", bf16=dtype == torch.bfloat16)


N_MM_FUZZ = 48


@pytest.mark.parametrize("case", range(N_MM_FUZZ), ids=lambda i: "mm-fuzz-%d" % i)
def test_random_shapes(case):
    """Seeded random M, N (1 .. 599), K (64 .. 2560), scale layout and C type:
    exact (bf16 C: the RNE rounding of the exact sum) where every partial sum
    is a binary32 number, within the accumulation bound otherwise."""
    rng = np.random.default_rng(7000 + case)
    M, N = int(rng.integers(1, 600)), int(rng.integers(1, 600))
    K = 64 * int(rng.integers(1, 41))
    layout = str(rng.choice(["row", "tiled"]))
    exact = bool(rng.integers(2)) and K <= 1024
    dtype = torch.float32 if rng.integers(2) else torch.bfloat16
    lo, hi = (126, 129) if exact else (100, 150)
    a, b = operand(rng, M, K, lo, hi), operand(rng, N, K, lo, hi)
    c, s = ref.mx_mm(*a, *b, M, N, K)
    got = gpu_mm(a, b, dtype=dtype, layout=layout)
    what = "M %d N %d K %d %s %s" % (M, N, K, layout, dtype)
    if exact and dtype == torch.float32:
        np.testing.assert_array_equal(got, c, err_msg=what)
    elif exact:
        want = ref.bf16_to_f32(ref.f32_to_bf16(c.astype(np.float32))).astype(np.float64)
        np.testing.assert_array_equal(got, want, err_msg=what)
    else:
        within_bound(got, c, s, K, what, bf16=dtype == torch.bfloat16)
