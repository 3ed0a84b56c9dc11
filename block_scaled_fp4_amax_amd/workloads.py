"""Seeded synthetic inputs for the five reference workloads.

This module draws inputs only; it holds none of the quantiser's arithmetic.
Samples are float32 from numpy's PCG64 generator, scaled in float32 and
rounded to bf16 by torch's cast (round to nearest even); tensors are returned
as uint16 bf16 bit patterns.  Both the HIP path and the CPU oracle are fed the
same arrays.

Shapes and value distributions follow the pages' workloads: hidden size 2880
and 32 MoE experts of 2880 x 2880 ("NVFP4 / AMD-FP4 outer-block (two-level)
scaling for FP4 training"), heavy-tailed outlier channels / tokens and
lognormal "massive activations" (same page, Background and Op-level tests),
an 8192 x 8192 bf16 weight ("MXFP4 weight QAT recipes", Implementations), and
its edge domains (+-0, 2^-127 / 2^-128 / 2^-133 subnormals, values near
6*2^125, inf and NaN poisoning, RTNE midpoints, scale-threshold triples;
same page, Correctness).  No model weights or datasets are used.
"""
import numpy as np
import torch


def to_bf16(f):
    """float32 array -> uint16 bf16 bits (torch cast, RNE)."""
    t = torch.from_numpy(np.ascontiguousarray(f, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def from_bf16(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------------ NVFP4 tensorwise QDQ, 256 x 256
def tensorwise_input_256(seed=0, rows=256, cols=256):
    """NVFP4 tensorwise QDQ input: N(0, 1)."""
    rng = np.random.default_rng(seed)
    return to_bf16(rng.standard_normal((rows, cols), dtype=np.float32))


# ------------------------------------------------------------------ NVFP4 2D-outer cast-transpose, 4096 x 4096
def weight_4096_outlier_cols(seed=2, rows=4096, cols=4096, outlier_frac=0.005, factor=1000.0):
    """Weight N(0, 0.02) with round(0.5% of cols) seeded columns scaled x1000."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(0.02)
    n_out = int(round(outlier_frac * cols))
    cols_out = rng.choice(cols, n_out, replace=False)
    w[:, cols_out] *= np.float32(factor)
    return to_bf16(w)


# ------------------------------------------------------------------ MXFP4 fake-quant, 8192 x 8192
TINY_BF16 = np.array([0x0000, 0x0040, 0x0020, 0x0001, 0x0060, 0x0080, 0x0100], np.uint16)
CAP_BF16 = np.array([0x7F3F, 0x7F40, 0x7F41], np.uint16)
MID_VALUES = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float32)


def mx_weight_8192_edges(seed=3, rows=8192, cols=8192, std=0.02):
    """MXFP4 fake-quant input: N(0, 0.02) with, in every group of 1024
    consecutive 1x32 blocks, ten seeded blocks rewritten: one single +-inf, one
    single NaN, one block of tiny values (+-0, 2^-127, 2^-128, 2^-133,
    3*2^-128, 2^-126, 2^-125), one cap block (first element 0x7F3F / 0x7F40 /
    0x7F41, i.e. around 6*2^125, rest N(0,1)*2^120), one block of E2M1
    midpoints and grid points scaled by 2^e with amax 6*2^e (e in [-20, 20]),
    one scale-threshold block whose amax is 6*2^k or one bf16 ulp either side,
    and four ordinary blocks sprinkled with +-0 and subnormals."""
    assert cols % 32 == 0 and (rows * cols // 32) % 1024 == 0
    rng = np.random.default_rng(seed)
    x = to_bf16(rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(std))
    blocks = x.reshape(-1, 32)
    G = blocks.shape[0] // 1024
    pick = np.argsort(rng.random((G, 1024), dtype=np.float32), axis=1)[:, :10].astype(np.int64)
    pick += (np.arange(G, dtype=np.int64) * 1024)[:, None]
    inf_b, nan_b, tiny_b, cap_b, mid_b, thr_b = (pick[:, k] for k in range(6))
    sprinkle = pick[:, 6:10].ravel()
    gi = np.arange(G)
    sgn = lambda shape: (rng.integers(0, 2, shape).astype(np.uint16) << 15)  # noqa: E731

    blocks[inf_b, rng.integers(0, 32, G)] = np.uint16(0x7F80) | sgn(G)
    blocks[nan_b, rng.integers(0, 32, G)] = 0x7FC0
    blocks[tiny_b] = rng.choice(TINY_BF16, (G, 32)) | sgn((G, 32))
    cap_rest = to_bf16(rng.standard_normal((G, 32), dtype=np.float32) * np.float32(2.0 ** 120))
    cap_rest[:, 0] = CAP_BF16[gi % 3] | sgn(G)
    blocks[cap_b] = cap_rest
    e = rng.integers(-20, 21, G)
    mids = rng.choice(MID_VALUES, (G, 32)) * np.exp2(e)[:, None].astype(np.float32)
    mids *= np.where(rng.integers(0, 2, (G, 32)) == 1, -1.0, 1.0).astype(np.float32)
    mids[:, 0] = np.float32(6.0) * np.exp2(e).astype(np.float32)
    blocks[mid_b] = to_bf16(mids)
    k = rng.integers(-20, 21, G)
    thr = to_bf16(np.clip(rng.standard_normal((G, 32), dtype=np.float32), -4, 4) * np.exp2(k)[:, None].astype(np.float32))
    six = to_bf16((np.float32(6.0) * np.exp2(k)).astype(np.float32)).astype(np.int64)
    thr[gi, rng.integers(0, 32, G)] = (six + rng.integers(-1, 2, G)).astype(np.uint16)
    blocks[thr_b] = thr
    spr_pos = rng.integers(0, 32, (sprinkle.size, 3))
    spr_val = rng.choice(np.array([0x0000, 0x0001, 0x0040, 0x0020], np.uint16), (sprinkle.size, 3))
    blocks[sprinkle[:, None], spr_pos] = spr_val | sgn((sprinkle.size, 3))
    return x


# ------------------------------------------------------------------ AMD-FP4 1D-outer SR cast-transpose, 16384 x 2880
def activations_16384x2880(seed=4, rows=16384, cols=2880, sigma=2.0, chan_frac=0.001, chan_factor=500.0):
    """Activations: N(0, 1) x per-token lognormal(0, 2) x500 on round(0.1% of
    cols) seeded channels."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((rows, cols), dtype=np.float32)
    a *= rng.lognormal(0.0, sigma, (rows, 1)).astype(np.float32)
    chans = rng.choice(cols, int(round(chan_frac * cols)), replace=False)
    a[:, chans] *= np.float32(chan_factor)
    return to_bf16(a)


# ------------------------------------------------------------------ grouped NVFP4 SR + EF, 32 x 2880 x 2880
def experts_32x2880(seed=5, experts=32, rows=2880, cols=2880, std=0.02, outlier_rows=2, factor=200.0):
    """Stacked MoE expert weights [experts * rows, cols]: N(0, 0.02), two seeded
    rows per expert x200."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((experts, rows, cols), dtype=np.float32) * np.float32(std)
    for e in range(experts):
        w[e, rng.choice(rows, outlier_rows, replace=False), :] *= np.float32(factor)
    return to_bf16(w.reshape(experts * rows, cols))


def expert_update(t, shape, std=1e-4):
    """Weight update of step t: N(0, 1e-4) float32, seeded 500 + t."""
    rng = np.random.default_rng(500 + t)
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def apply_expert_update(w_bits, dw):
    """W_{t+1} = bf16(f32(W_t) + dW_t); independent of the quantiser output."""
    return to_bf16(from_bf16(w_bits) + dw)



# ------------------------------------------------------------------ binary32 sources
def fp32_weights(seed, rows, cols, std=0.02):
    """A binary32 source with full 24-bit significands: N(0, std) x per-row
    lognormal(0, 2), one seeded row x300, one seeded column x1e-3, seeded
    signed zeros and binary32 subnormals (float32 array; no inf / NaN)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(std)
    x *= rng.lognormal(0.0, 2.0, (rows, 1)).astype(np.float32)
    x[rng.integers(0, rows), :] *= np.float32(300)
    x[:, rng.integers(0, cols)] *= np.float32(1e-3)
    n = rows * cols
    k = max(1, n // 512)
    x.ravel()[rng.integers(0, n, k)] = 0.0
    x.ravel()[rng.integers(0, n, k)] = -0.0
    sub = rng.integers(1, 1 << 23, k, dtype=np.uint64).astype(np.uint32)
    sub |= rng.integers(0, 2, k, dtype=np.uint64).astype(np.uint32) << np.uint32(31)
    x.ravel()[rng.integers(0, n, k)] = sub.view(np.float32)
    return x


def fp32_raw_bit_blocks(seed, rows, cols):
    """Raw binary32 bit patterns in 1 x 32 blocks (uint32): every fourth block
    uniformly random bits (NaN / inf / subnormal patterns included), the others
    random significands and signs within one to four binades drawn per block,
    or binary32 subnormals."""
    rng = np.random.default_rng(seed)
    x = np.zeros((rows, cols), np.uint32)
    for i in range(rows):
        for j0 in range(0, cols, 32):
            kind = (i * (cols // 32) + j0 // 32) % 4
            raw = rng.integers(0, 1 << 32, 32, dtype=np.uint64).astype(np.uint32)
            if kind == 0:
                x[i, j0:j0 + 32] = raw
                continue
            e = int(rng.integers(1, 250)) if kind != 3 else 0
            span = int(rng.integers(0, 4))
            exps = (e + (raw >> np.uint32(24)) % np.uint32(span + 1)) if kind != 3 else np.zeros(32, np.uint32)
            x[i, j0:j0 + 32] = (raw & np.uint32(0x807FFFFF)) | (exps.astype(np.uint32) << np.uint32(23))
    return x


CONFIGS = {
    "nv_tensorwise_qdq_256": dict(name="nvfp4_tensorwise_qdq_256x256", rows=256, cols=256),
    "nv_2d_cast_transpose_4096": dict(name="nvfp4_outer2d64_cast_transpose_4096x4096", rows=4096, cols=4096),
    "mx_fake_quant_8192": dict(name="mxfp4_fake_quant_8192x8192", rows=8192, cols=8192),
    "amd_1d_sr_cast_transpose_16384x2880": dict(name="amdfp4_outer1d64_sr_cast_transpose_16384x2880", rows=16384, cols=2880),
    "nv_grouped_sr_ef_32x2880": dict(name="nvfp4_grouped32_outer2d64_sr_ef_2880x2880", rows=32 * 2880, cols=2880),
}
