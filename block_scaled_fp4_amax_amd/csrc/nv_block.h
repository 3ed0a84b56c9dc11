// nv_block.h -- per-16-element NVFP4 / AMD-FP4 inner quantisation shared by the
// rowwise and tile kernels (device only).
//
// "fp4-train" README, Method: a block's scale is block_absmax / 6 encoded on
// the inner grid (E4M3, or UE5M3 for AMD-FP4 -- "NVFP4 / AMD-FP4 outer-block
// (two-level) scaling", Background); every element is divided by the decoded
// scale and rounded onto the E2M1 grid, to nearest-even or stochastically.
#pragma once

#include "fp4q_device.h"

namespace fp4q {

// RN64(1 / d) for every decoded inner scale d, from a 16-entry table of the
// reciprocals of the 3-bit significands: d = (1 + m/8) * 2^(e - BIAS) for
// e >= 1 and d = (m / 8) * 2^(1 - BIAS) for e == 0; entry 8 (d == 0) is 0, so
// a zero scale yields quotients of (signed) zero.  Exact power-of-two scaling
// of a binary64 value commutes with its rounding, so the result is RN64(1/d).
constexpr int kRecipTableSize = 16;

// Entries m = 0..7: RN64(1 / (1 + m/8)); 8: 0; 9..15: RN64(8 / (m - 8)).
// Each quotient is a constant expression, evaluated by the compiler as one
// correctly rounded binary64 division.
constexpr double kRecipTable[16] = {
    1.0 / 1.0, 1.0 / 1.125, 1.0 / 1.25, 1.0 / 1.375, 1.0 / 1.5, 1.0 / 1.625, 1.0 / 1.75, 1.0 / 1.875,
    0.0, 8.0 / 1.0, 8.0 / 2.0, 8.0 / 3.0, 8.0 / 4.0, 8.0 / 5.0, 8.0 / 6.0, 8.0 / 7.0};

__device__ __forceinline__ void fill_recip_table(double* t, int lane)
{
    double v = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) v = lane == i ? kRecipTable[i] : v;
    if (lane < 16) t[lane] = v;
}

template <int BIAS>
__device__ __forceinline__ double inner_recip(uint32_t code, const double* tab)
{
    const uint32_t e = code >> 3, m = code & 7u;
    const uint32_t idx = m | (e == 0u ? 8u : 0u);
    const int sh = BIAS - (int)(e == 0u ? 1u : e);
    return ldexp(tab[idx], sh);
}

// Scale of one block from its max |v_n|: code, decoded value, RN64(1/d).
template <int BIAS>
struct BlockScale {
    uint32_t code;
    float d;
    double rd;
};

template <int BIAS>
__device__ __forceinline__ BlockScale<BIAS> block_scale(float bmax, const double* tab)
{
    BlockScale<BIAS> s;
    // RN32(bmax / 6): any quotient below the normal range encodes to code 0
    // either way (the smallest nonzero inner scale is far above it).
    const float y = div_inv64(bmax, 1.0 / 6.0);
    constexpr float kMax = BIAS == 7 ? 448.0f : 114688.0f;
    constexpr uint32_t kMaxCode = BIAS == 7 ? 0x7Eu : 0xFEu;
    constexpr float kMinNormal = BIAS == 7 ? 0x1p-6f : 0x1p-14f;
    constexpr float kToSteps = BIAS == 7 ? 0x1p9f : 0x1p17f;      // subnormal grid step 2^-(BIAS+2)
    constexpr float kFromSteps = BIAS == 7 ? 0x1p-9f : 0x1p-17f;
    // normal range (the common case): round to nearest even at 3 mantissa
    // bits on the bit pattern; RN64(1 / d) is the table entry of the 3-bit
    // significand times 2^-(exponent of d)
    const uint32_t u = __float_as_uint(y);
    const uint32_t un = (u + 0x7FFFFu + ((u >> 20) & 1u)) & 0xFFF00000u;
    s.code = (un >> 20) - ((127u - (uint32_t)BIAS) << 3);
    s.d = __uint_as_float(un);
    s.rd = ldexp(tab[(un >> 20) & 7u], 127 - (int)(un >> 23));
    if (!(y >= kMinNormal && y < kMax)) {
        // saturated, or below the normal range: a whole number of subnormal
        // grid steps, 0..8 (8 is the smallest normal)
        const float steps = __builtin_rintf(y * kToSteps);
        const bool sat = y >= kMax;
        s.code = sat ? kMaxCode : (uint32_t)steps;
        s.d = sat ? kMax : steps * kFromSteps;
        s.rd = inner_recip<BIAS>(s.code, tab);
    }
    return s;
}

__device__ __forceinline__ float max_abs16(const float (&v)[16])
{
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) m = fmaxf(m, __builtin_fabsf(v[k]));
    return m;
}

// ---------------------------------------------------------------- RNE codes without a division
// The RNE code of t = RN32(v / d) depends only on where v / d lies relative to
// the binary32 rounding boundaries B next to the E2M1 decision points
// 0.25, 0.75, 1.25, 1.75, 2.5, 3.5 and 5 (B = point +- half an ulp; ties at B
// round to the point, whose last significand bit is 0).  Write d = D 2^E with
// D in 8..15.  In units of 2^(e - 25) (e the decision point's exponent) B is
// an integer with at most one factor 2, so v / d = B would need a factor 16 in
// D (D = 8 divides exactly anyway); otherwise v (24 significant bits) is at
// least one such unit times d away from B d, so |v / d - B| >= 2^-30 |v / d|.
// With Kh = RD32(1 / D) 2^-E (rounded down) and Kl = RN32(1 / D - RD32(1 / D)) 2^-E
// (so Kl >= 0 and v Kh and v Kl share the sign of v, which keeps -0 a -0),
// u = v Kh + RN32(v Kl) is within 2^-46 |v / d| of v / d, on the same side of
// every B, so RN32(u) (one fused multiply-add) has the same code as t: one
// multiply and one fma per value instead of a binary64 product.  Zero scale:
// Kh = Kl = 0 gives signed zeros, as t does.  Results far below 0.25 (code 0,
// sign kept) are exact either way.  The table holds (Kh, Kl) per scale code.
constexpr int kRneTableSize = 256;

template <int BIAS>
__device__ __forceinline__ void fill_rne_table(float2* tab, int code)
{
    // RD32(1 / D) and RN32(1 / D - RD32(1 / D)) for D = 8..15
    constexpr float kh[8] = {0x1p-3f, 0x1.c71c7p-4f, 0x1.999998p-4f, 0x1.745d16p-4f,
                             0x1.555554p-4f, 0x1.3b13bp-4f, 0x1.249248p-4f, 0x1.11111p-4f};
    constexpr float kl[8] = {0.0f, 0x1.c71c72p-28f, 0x1.99999ap-28f, 0x1.45d174p-28f,
                             0x1.555556p-28f, 0x1.3b13b2p-28f, 0x1.24924ap-28f, 0x1.111112p-28f};
    if (code >= kRneTableSize) return;
    const float d = code <= (int)ScaleFmt<BIAS>::max_code ? scale_decode<BIAS>((uint32_t)code) : 0.0f;
    const uint32_t bd = __float_as_uint(d);
    const int m = (int)((bd >> 20) & 7u);                // D = 8 + m
    const int e = (int)(bd >> 23) - 127 - 3;              // d = D 2^e
    float h = 0.0f, l = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        h = m == i ? kh[i] : h;
        l = m == i ? kl[i] : l;
    }
    tab[code] = d == 0.0f ? make_float2(0.0f, 0.0f) : make_float2(ldexpf(h, -e), ldexpf(l, -e));
}

// RNE codes of 16 normalised values: t = RN32(v_n / d) through the table entry
// k = (Kh, Kl) of the block's scale code, then the hardware E2M1 pack.
__device__ __forceinline__ uint2 codes16_rne(const float (&vn)[16], float2 k)
{
    float t[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) t[i] = __builtin_fmaf(vn[i], k.x, vn[i] * k.y);
    uint32_t lo = 0, hi = 0;
    lo = fp4x2_rne<0>(lo, t[0], t[1]);
    lo = fp4x2_rne<1>(lo, t[2], t[3]);
    lo = fp4x2_rne<2>(lo, t[4], t[5]);
    lo = fp4x2_rne<3>(lo, t[6], t[7]);
    hi = fp4x2_rne<0>(hi, t[8], t[9]);
    hi = fp4x2_rne<1>(hi, t[10], t[11]);
    hi = fp4x2_rne<2>(hi, t[12], t[13]);
    hi = fp4x2_rne<3>(hi, t[14], t[15]);
    return make_uint2(lo, hi);
}

// ---------------------------------------------------------------- stochastic-rounding codes
// Stochastic rounding of t = RN32(|v_n| / d) onto the E2M1 grid ("fp4-train"
// README, Method): between neighbours lo < hi round up iff u16 < frac * 2^16,
// frac = (t - lo) / (hi - lo), with grid points and t >= 6 deterministic.
//
// gfx950's v_cvt_scalef32_sr_pk_fp4_f32 does this in one instruction once its
// inputs are arranged (every case checked on the device: all 65536 u16 against
// about 3100 t values covering every binade, the fractions next to each k/2^16
// and the subnormal range).  Measured behaviour of the instruction with the
// value in its first slot: it sees t on a grid of 2^-23 (below 1, lower bits of
// t are dropped), and rounds up iff the 22 bits of t's fraction below the E2M1
// step plus the top 22 bits of the seed carry.  So:
//   - the value passed is c = ceil(t * 2^23) with the instruction's exact
//     power-of-two scale 2^23 (t' = c / 2^23; for t >= 1, t' = t): rounding a
//     dropped remainder up makes "u16 < frac * 2^16" and "carry" agree for
//     every fraction, since u16 * 2^(k-16) and the kept bits are multiples of
//     the grid step;
//   - seed = (~u16 << 16) | 0xFFFF: its top 22 bits are 2^22 - 1 - 64 u16, so
//     the carry happens iff the kept fraction exceeds 64 u16;
//   - the instruction's second slot draws from the seed shifted by one bit, so
//     each element goes through a first slot of its own: even elements into one
//     word, odd elements into another, merged by a shift.
// c = ceil(T - 2^-127) with T = |v_n| / d * 2^23 rounded to binary32: that is
// t * 2^23 exactly while t is a normal binary32.  Below that only "t > 0"
// matters (c = 1 rounds up iff u16 == 0), and t > 0 exactly when T > 2^-127:
// the quotient v_n / d is either 2^-150 exactly (T = 2^-127, t = 0) or at
// least 2^-7 of itself away from it (v_n is then subnormal and d has 4
// significant bits).  ceil(T - 2^-127) gives both cases, and ceil(t * 2^23)
// from T = 2^-100 on.  T comes from the scale code's two-term reciprocal (the
// RNE table below, times 2^23): with d of at most 4 significant bits, |v_n| / d
// is never within 2^-29 (relative) of a binary32 rounding midpoint, and
// |v_n| Kh + RN32(|v_n| Kl) is within 2^-46 of it, so one fma rounds it to the
// same binary32; the -2^-127 rides in the low term (it is below half an ulp of
// T from T = 2^-103 on, and below that only T's side of 2^-127 matters, which
// it keeps).  Two fmas and a ceil per value, checked on the CPU against
// ceil(RN32(|v_n| RN64(1/d) 2^23) - 2^-127) for every scale code of both inner
// formats on 3.2e8 values (log-uniform over 2^-160 .. 2^8 times d, the
// neighbourhoods of decision points, and the subnormal range), each with and
// without the clamp.  Without an outer scale t can exceed 2^104 (saturated inner
// scales), so CLAMP bounds T to [0, 6 * 2^23]; otherwise t stays near 6 and the
// instruction saturates by itself.  Magnitude nibbles carry no sign (the masks
// drop the -0 that ceil gives for T < 0); the sign nibbles come from the
// hardware RNE pack of v_n / 2^125, which is a zero of v_n's sign unless
// |v_n| >= 2^123, and such values saturate (code 7) under every inner scale,
// so OR-ing stays exact.

// The code of c / 2^23 (first slot, seed as above) into byte SEL of acc, the
// other bytes kept: the instruction writes only the selected byte, its
// destination being also its input.  The builtin for it does not tie that
// input to the destination (the byte-select form would leave the other bytes
// undefined), so the instruction is written out with the accumulator as a
// read-write operand; the compiler pads what follows it for the partial-write
// forwarding hazard as for any inline asm.  The second slot holds +0, whose
// code is 0, so byte SEL becomes the element's code in its low nibble; the
// only stray bit is the sign of a -0 (ceil of a negative T), which one mask
// per word removes.
template <int SEL>
__device__ __forceinline__ void sr_code_into(uint32_t& acc, float c, uint32_t seed)
{
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    f32x2_t v;
    v.x = c;
    v.y = 0.0f;
    if constexpr (SEL == 0)
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3" : "+v"(acc) : "v"(v), "v"(seed), "s"(0x1p23f));
    else if constexpr (SEL == 1)
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,1,0]" : "+v"(acc) : "v"(v), "v"(seed),
            "s"(0x1p23f));
    else if constexpr (SEL == 2)
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,0,1]" : "+v"(acc) : "v"(v), "v"(seed),
            "s"(0x1p23f));
    else
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,1,1]" : "+v"(acc) : "v"(v), "v"(seed),
            "s"(0x1p23f));
}

// The seed (~u16 << 16) | 0xFFFF of the variate in the low half of w (the high
// half ignored) in one instruction: v_mad_i32_i24 takes w's low 24 bits as a
// signed number, and times -2^16 its bits 16..23 only add multiples of 2^32, so
// the result is -2^16 u16 - 1 = ~(u16 << 16) modulo 2^32.  (Written out: the
// compiler turns the plain expression into a shift and a not.)
__device__ __forceinline__ uint32_t sr_seed_lo(uint32_t w)
{
    uint32_t s;
    asm("v_mad_i32_i24 %0, %1, %2, -1" : "=v"(s) : "v"(w), "s"(-65536));
    return s;
}

// The seed of the variate in the high half of w: ~w | 0xFFFF.
__device__ __forceinline__ uint32_t sr_seed_hi(uint32_t w)
{
    return ~w | 0xFFFFu;
}

// ceil(|v| / d * 2^23 - 2^-127) from (Kh, Kl) * 2^23 of the block's scale.
template <bool CLAMP>
__device__ __forceinline__ float sr_fixed23(float v, float kh23, float kl23)
{
    const float av = __builtin_fabsf(v);
    float a = __builtin_fmaf(av, kh23, __builtin_fmaf(av, kl23, -0x1p-127f));
    if (CLAMP) a = __builtin_amdgcn_fmed3f(a, 0.0f, 0x1.8p25f);
    return __builtin_ceilf(a);
}

// Eight SR codes; seed(k) gives element k's seed.  Even elements go to the
// bytes of one word, odd ones to another, merged by a shift.
template <bool CLAMP, class Seed>
__device__ __forceinline__ uint32_t codes8_sr(const float* vn, Seed seed, float kh23, float kl23)
{
    constexpr float kSignOnly = 0x1p125f;
    uint32_t sg = 0;
    sg = fp4x2_rne_scaled<0>(sg, vn[0], vn[1], kSignOnly);
    sg = fp4x2_rne_scaled<1>(sg, vn[2], vn[3], kSignOnly);
    sg = fp4x2_rne_scaled<2>(sg, vn[4], vn[5], kSignOnly);
    sg = fp4x2_rne_scaled<3>(sg, vn[6], vn[7], kSignOnly);
    uint32_t ev = 0, od = 0;
    sr_code_into<0>(ev, sr_fixed23<CLAMP>(vn[0], kh23, kl23), seed(0));
    sr_code_into<0>(od, sr_fixed23<CLAMP>(vn[1], kh23, kl23), seed(1));
    sr_code_into<1>(ev, sr_fixed23<CLAMP>(vn[2], kh23, kl23), seed(2));
    sr_code_into<1>(od, sr_fixed23<CLAMP>(vn[3], kh23, kl23), seed(3));
    sr_code_into<2>(ev, sr_fixed23<CLAMP>(vn[4], kh23, kl23), seed(4));
    sr_code_into<2>(od, sr_fixed23<CLAMP>(vn[5], kh23, kl23), seed(5));
    sr_code_into<3>(ev, sr_fixed23<CLAMP>(vn[6], kh23, kl23), seed(6));
    sr_code_into<3>(od, sr_fixed23<CLAMP>(vn[7], kh23, kl23), seed(7));
    return sg | (ev & 0x07070707u) | ((od & 0x07070707u) << 4);
}

// SR codes of 16 normalised values with the block's scale, given as its RNE
// table entry k = (Kh, Kl); CLAMP when no outer scale bounds the quotients.
// Variates packed two per word: element k's is bits 16 (k & 1) .. + 15 of u[k >> 1].
template <bool CLAMP>
__device__ __forceinline__ uint2 codes16_sr(const float (&vn)[16], const uint32_t (&u)[8], float2 k)
{
    const float kh23 = k.x * 0x1p23f, kl23 = k.y * 0x1p23f;
    auto lo_seed = [&](int e) { return (e & 1) ? sr_seed_hi(u[e >> 1]) : sr_seed_lo(u[e >> 1]); };
    auto hi_seed = [&](int e) { return (e & 1) ? sr_seed_hi(u[4 + (e >> 1)]) : sr_seed_lo(u[4 + (e >> 1)]); };
    const uint32_t lo = codes8_sr<CLAMP>(vn, lo_seed, kh23, kl23);
    const uint32_t hi = codes8_sr<CLAMP>(vn + 8, hi_seed, kh23, kl23);
    return make_uint2(lo, hi);
}

// The same with one variate per word (element k's in the low half of u[k]).
template <bool CLAMP>
__device__ __forceinline__ uint2 codes16_sr(const float (&vn)[16], const uint32_t (&u)[16], float2 k)
{
    const float kh23 = k.x * 0x1p23f, kl23 = k.y * 0x1p23f;
    auto lo_seed = [&](int e) { return sr_seed_lo(u[e]); };
    auto hi_seed = [&](int e) { return sr_seed_lo(u[8 + e]); };
    const uint32_t lo = codes8_sr<CLAMP>(vn, lo_seed, kh23, kl23);
    const uint32_t hi = codes8_sr<CLAMP>(vn + 8, hi_seed, kh23, kl23);
    return make_uint2(lo, hi);
}

// Signed inner-dequantised values p = +-G[m] * d from 16 packed codes (the
// hardware E2M1 decode at scale 1, then an exact product with d).
template <int Q>
__device__ __forceinline__ void decode_byte(uint32_t w, float d, float& a, float& b)
{
    auto f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, Q);
    a = f[0] * d;
    b = f[1] * d;
}

__device__ __forceinline__ void decode16(uint2 packed, float d, float (&p)[16])
{
    decode_byte<0>(packed.x, d, p[0], p[1]);
    decode_byte<1>(packed.x, d, p[2], p[3]);
    decode_byte<2>(packed.x, d, p[4], p[5]);
    decode_byte<3>(packed.x, d, p[6], p[7]);
    decode_byte<0>(packed.y, d, p[8], p[9]);
    decode_byte<1>(packed.y, d, p[10], p[11]);
    decode_byte<2>(packed.y, d, p[12], p[13]);
    decode_byte<3>(packed.y, d, p[14], p[15]);
}

// Normalise by an outer scale: v_n = RN32(v / s_o), v_n = +-0 when s_o == 0.
// inv = RN64(1 / s_o) (0 when s_o == 0).
// - The reciprocal product RN32(v inv) is exact for normal-range quotients:
//   there v / s_o is at least 2^-49 of itself away from every binary32
//   rounding midpoint.
// - Below the normal range a quotient can be an exact midpoint of the
//   subnormal grid, which the product may round past (for example
//   s_o = 49 * 2^18 and v = 147 * 2^-132: 2^-149 against 2^-148). Such
//   quotients are recomputed by binary32 division.
// - Only stochastic rounding needs this (RECHECK). A subnormal v_n is below
//   2^-109 times every nonzero inner scale (the smallest is 2^-17, UE5M3), so
//   its RNE code is 0 whatever its value. A block whose largest v_n is subnormal encodes a zero scale either
//   way, and the dequantised value and residual follow from code, scale and
//   s_o alone. Under stochastic rounding, whether t = RN32(v_n / d) is nonzero
//   decides if a variate of 0 rounds up.
// - A lane can have a subnormal quotient only if min |v| 2^126 < s_o. The
//   scaling is exact, or overflows for |v| >= 4 where no quotient is subnormal.
//   Only when that holds in some lane of the wave (a wave-uniform branch) are
//   the results tested one by one. For bf16 values (BF16: no residual was
//   added) |v| >= 2^-133 rules it out while s_o <= 2^-7, so the minimum is
//   taken only in waves where some lane's scale is larger.
constexpr float kNoSubnormalScale = 0x1p-7f;

template <bool RECHECK, bool BF16>
__device__ __forceinline__ void normalize16(const float (&v)[16], float s_o, double inv, float (&vn)[16])
{
#pragma unroll
    for (int k = 0; k < 16; ++k) vn[k] = div_inv64(v[k], inv);
    if (!RECHECK) return;
    if (BF16 && __builtin_amdgcn_ballot_w64(!(s_o <= kNoSubnormalScale)) == 0) return;
    float m = __builtin_fabsf(v[0]);
#pragma unroll
    for (int k = 1; k < 16; ++k) m = fminf(m, __builtin_fabsf(v[k]));
    bool slow = false;
    if (__builtin_amdgcn_ballot_w64(m * 0x1p126f < s_o) != 0) {
#pragma unroll
        for (int k = 0; k < 16; ++k) slow |= is_subnormal(vn[k]);
    }
    if (__builtin_expect(slow, 0)) {
#pragma unroll
        for (int k = 0; k < 16; ++k)
            if (is_subnormal(vn[k])) vn[k] = v[k] / s_o;
    }
}

// Outer scale RN32(amax / den) for den = scale_max * 6 (2688 or 688128).
__device__ __forceinline__ float outer_scale(float amax, float den)
{
    float s = div_inv64(amax, 1.0 / (double)den);
    if (__builtin_expect(is_subnormal(s), 0)) s = amax / den;
    return s;
}

__device__ __forceinline__ double outer_inv(float s_o)
{
    return s_o == 0.0f ? 0.0 : 1.0 / (double)s_o;
}

}  // namespace fp4q
