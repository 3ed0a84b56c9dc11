// fp4q_device.h -- device-side number formats for the gfx950 kernels.
//
// Everything here is bit-level integer work or single IEEE binary32
// operations (the build uses -ffp-contract=off, correctly rounded fp32
// division and no denormal flushing), so each helper computes exactly the
// binary32 result its comment names.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4q {

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// binary32 -> bf16 bits, round to nearest even; any NaN -> 0x7FC0
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------- E2M1
// Magnitude code (0..7 on {0, .5, 1, 1.5, 2, 3, 4, 6}) of t >= 0 by round to
// nearest, ties to the even code, saturating at 6 ("fp4-train" README, Method;
// "MXFP4 weight QAT recipes", Correctness: RTNE midpoints, satfinite).
// The midpoints between neighbours are 0.25, 0.75, 1.25, 1.75, 2.5, 3.5 and 5;
// a tie goes up exactly where the upper neighbour has the even code.
__device__ __forceinline__ uint32_t e2m1_rne(float t)
{
    return (uint32_t)(t > 0.25f) + (uint32_t)(t >= 0.75f) + (uint32_t)(t > 1.25f) + (uint32_t)(t >= 1.75f) +
           (uint32_t)(t > 2.5f) + (uint32_t)(t >= 3.5f) + (uint32_t)(t > 5.0f);
}

__device__ __forceinline__ float e2m1_value(uint32_t m)
{
    // {0, .5, 1, 1.5, 2, 3, 4, 6}: m < 2 -> m/2; else (1 + (m&1)/2) * 2^((m>>1)-1)
    float lo = 0.5f * (float)m;
    float hi = __uint_as_float(((127u + (m >> 1) - 1u) << 23) | ((m & 1u) << 22));
    return m < 2u ? lo : hi;
}

// Stochastic rounding of t >= 0 onto the grid: between neighbours lo < hi the
// result is hi with probability (t - lo) / (hi - lo), realised as
// u16 < frac * 2^16 with u16 uniform in [0, 2^16) ("fp4-train" README,
// Method).  Grid points and t >= 6 are deterministic.
__device__ __forceinline__ uint32_t e2m1_sr(float t, uint32_t u16)
{
    if (t >= 6.0f) return 7u;
    uint32_t lo = (uint32_t)(t >= 0.5f) + (uint32_t)(t >= 1.0f) + (uint32_t)(t >= 1.5f) + (uint32_t)(t >= 2.0f) +
                  (uint32_t)(t >= 3.0f) + (uint32_t)(t >= 4.0f);
    float g = e2m1_value(lo);
    // gap to the next grid point: 0.5 below 2, 1 in [2, 4), 2 in [4, 6)
    float inv_gap = lo < 4u ? 2.0f : (lo < 6u ? 1.0f : 0.5f);
    float frac = (t - g) * inv_gap;            // exact (Sterbenz / power-of-two scaling)
    return lo + (uint32_t)((float)u16 < frac * 65536.0f);
}

// ---------------------------------------------------------------- inner scale grids
// E4M3 (bias 7, max 448, subnormal step 2^-9) and UE5M3 (bias 15, max 114688,
// subnormal step 2^-17): 3 mantissa bits, top code reserved for NaN.
template <int BIAS> struct ScaleFmt {
    static constexpr uint32_t max_code = BIAS == 7 ? 0x7Eu : 0xFEu;
    static __device__ __forceinline__ float max_value() { return BIAS == 7 ? 448.0f : 114688.0f; }
    // outer denominator scale_max * 6 (ALTO page, Technical design)
    static __device__ __forceinline__ float outer_den() { return BIAS == 7 ? 2688.0f : 688128.0f; }
};

// RNE of y >= 0 onto the grid, satfinite, underflow to code 0.
template <int BIAS>
__device__ __forceinline__ uint32_t scale_encode(float y)
{
    if (y >= ScaleFmt<BIAS>::max_value()) return ScaleFmt<BIAS>::max_code;
    const float min_normal = __uint_as_float((uint32_t)(127 + 1 - BIAS) << 23);
    if (y < min_normal) {
        // subnormal step 2^(1-BIAS-3): scale to integer steps (exact), round half even
        const float to_steps = __uint_as_float((uint32_t)(127 + BIAS + 2) << 23);
        return (uint32_t)__builtin_rintf(y * to_steps);     // 0..8; 8 is the smallest normal code
    }
    uint32_t u = __float_as_uint(y);
    u = u + 0x7FFFFu + ((u >> 20) & 1u);                    // RNE to 3 mantissa bits
    uint32_t e = (u >> 23) - 127u + (uint32_t)BIAS;
    return (e << 3) | ((u >> 20) & 7u);
}

template <int BIAS>
__device__ __forceinline__ float scale_decode(uint32_t c)
{
    uint32_t e = c >> 3, m = c & 7u;
    const float sub_step = __uint_as_float((uint32_t)(127 + 1 - BIAS - 3) << 23);
    float sub = (float)m * sub_step;
    float nrm = __uint_as_float(((e + 127u - (uint32_t)BIAS) << 23) | (m << 20));
    return e == 0u ? sub : nrm;
}

// ---------------------------------------------------------------- Philox4x32-10
// Salmon et al., SC'11: ten rounds of two 32x32->64 multiplies with Feistel
// style mixing; the key is bumped by the Weyl constants between rounds.
struct u32x4 { uint32_t x, y, z, w; };

__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
        u32x4 n;
        n.x = (uint32_t)(p1 >> 32) ^ c.y ^ k0;
        n.y = (uint32_t)p1;
        n.z = (uint32_t)(p0 >> 32) ^ c.w ^ k1;
        n.w = (uint32_t)p0;
        c = n;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

// The eight 16-bit variates of elements 8*blk .. 8*blk+7: counter
// (lo32 blk, hi32 blk, lo32 step, hi32 step), key (lo32 seed, hi32 seed);
// element 8*blk + l takes 16-bit half (l & 1) of output word (l >> 1).
__device__ __forceinline__ u32x4 sr_words(uint64_t seed, uint64_t step, uint64_t blk)
{
    u32x4 c = {(uint32_t)blk, (uint32_t)(blk >> 32), (uint32_t)step, (uint32_t)(step >> 32)};
    return philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
}

__device__ __forceinline__ uint32_t sr_lane(const u32x4& w, int l)
{
    uint32_t word = (l >> 1) == 0 ? w.x : (l >> 1) == 1 ? w.y : (l >> 1) == 2 ? w.z : w.w;
    return (l & 1) ? (word >> 16) : (word & 0xFFFFu);
}

// ---------------------------------------------------------------- sanitisation
// NaN -> +0, +-inf -> +-largest finite bf16 (0x7F7F), applied to the value
// being quantised (NVFP4 / AMDFP4 paths).
__device__ __forceinline__ float sanitize(float v)
{
    uint32_t u = __float_as_uint(v);
    uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return 0.0f;
    if (a == 0x7F800000u) return __uint_as_float((u & 0x80000000u) | 0x7F7F0000u);
    return v;
}

// ---------------------------------------------------------------- cross-lane max
// Max over aligned groups of W consecutive lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_max(float v)
{
#pragma unroll
    for (int m = 1; m < W; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}

template <int W>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v)
{
#pragma unroll
    for (int m = 1; m < W; m <<= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)v, m, 64);
        v = v > o ? v : o;
    }
    return v;
}

}  // namespace fp4q
