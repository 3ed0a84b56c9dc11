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

// Two E2M1 codes (RNE, ties to the even code, saturating at 6, sign kept,
// signed zero kept) of a and b, written into byte SEL of `old` (a in the low
// nibble).  This is gfx950's v_cvt_scalef32_pk_fp4_f32 with scale 1; its
// rounding equals e2m1_rne() above on every non-negative binary32 (checked
// exhaustively on the device, together with the sign of every negative).
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_rne(uint32_t old, float a, float b)
{
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// Same with a power-of-two scale 2^k: codes of a / 2^k and b / 2^k, exact for
// every finite bf16 a, b and k in [-126, 125] (checked on the device).
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_rne_scaled(uint32_t old, float a, float b, float pow2)
{
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, pow2, SEL);
}

// ---------------------------------------------------------------- exact division
// RN32(a / s) computed as RN32(a * RN64(1 / s)).  For binary32 a and s the
// exact quotient is never a binary32 rounding midpoint (a midpoint has an odd
// 25-bit significand, which a * (odd part of s)^-1 cannot produce), and its
// distance to the nearest midpoint is at least 2^-49 of its magnitude, while
// a * RN64(1/s) rounded to binary64 is within 2^-52 of a / s.  So the binary32
// rounding of the binary64 product equals the correctly rounded quotient
// whenever that quotient is a normal binary32; callers route the few
// subnormal-range quotients through the IEEE division instead.  Signs and
// signed zeros carry through exactly.
__device__ __forceinline__ float div_inv64(float a, double inv)
{
    return (float)((double)a * inv);
}

// True when q is a subnormal binary32 (one v_cmp_class).  div_inv64 is exact
// for normal-range quotients; below that only an exact rounding tie of the
// quotient can round differently, and then the binary64 route lands on a
// subnormal neighbour (or on zero where zero is the correct result), so
// flagging subnormal results is enough to catch every such case.
__device__ __forceinline__ bool is_subnormal(float q)
{
    // The binary32 form of the class test: the unsuffixed builtin takes a
    // binary64 operand, and a widened binary32 is never a binary64 denormal,
    // so that form folds to false.
    return __builtin_amdgcn_classf(q, 0x090);   // -denormal | +denormal
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

// a ^ b ^ c in one instruction (gfx950's three-input bitwise operation;
// truth table 0x96 is the three-way exclusive or).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c)
{
    return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1)
{
    // The round keys are formed here, two scalar adds per round, rather than
    // hoisted out of the caller's loop as twenty loop-invariant scalars that
    // would overflow the scalar register file (and be spilled to vector lanes).
    asm volatile("" : "+s"(k0), "+s"(k1));
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
        u32x4 n;
        n.x = xor3(c.y, k0, (uint32_t)(p1 >> 32));
        n.y = (uint32_t)p1;
        n.z = xor3(c.w, k1, (uint32_t)(p0 >> 32));
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
// Element indices are taken modulo 2^64, so an element's counter is its wrapped
// index >> 3, below 2^61.  Callers form blk from a base and offsets without
// wrapping; it is congruent to the counter modulo 2^61 and reduced here.
__device__ __forceinline__ u32x4 sr_words(uint64_t seed, uint64_t step, uint64_t blk)
{
    blk &= (uint64_t(1) << 61) - 1;
    u32x4 c = {(uint32_t)blk, (uint32_t)(blk >> 32), (uint32_t)step, (uint32_t)(step >> 32)};
    return philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
}

__device__ __forceinline__ uint32_t sr_lane(const u32x4& w, int l)
{
    uint32_t word = (l >> 1) == 0 ? w.x : (l >> 1) == 1 ? w.y : (l >> 1) == 2 ? w.z : w.w;
    return (l & 1) ? (word >> 16) : (word & 0xFFFFu);
}

// The 16 SR variates of elements idx0 .. idx0+15 (idx0 = global index of the
// block's first element), packed two per word: element k's variate is bits
// 16*(k&1) .. 16*(k&1)+15 of u[k >> 1].  idx0 % 8 equals index_base % 8 for
// every block of a launch (blocks start at multiples of 16), so the branch is
// uniform; in the aligned case the eight Philox output words of the two
// 8-element counters are the packed variates themselves.
//
// The core takes the first 8-element counter b0 = idx0 >> 3 and off = idx0 % 8.
__device__ __forceinline__ void sr_draws16_at(uint64_t seed, uint64_t step, uint64_t b0, int off, uint32_t (&u)[8])
{
    const u32x4 w0 = sr_words(seed, step, b0);
    const u32x4 w1 = sr_words(seed, step, b0 + 1);
    if (off == 0) {
        u[0] = w0.x; u[1] = w0.y; u[2] = w0.z; u[3] = w0.w;
        u[4] = w1.x; u[5] = w1.y; u[6] = w1.z; u[7] = w1.w;
    } else {
        const u32x4 w2 = sr_words(seed, step, b0 + 2);
        uint32_t e16[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int e = off + k;
            const int blk = e >> 3;
            u32x4 w;
            w.x = blk == 0 ? w0.x : (blk == 1 ? w1.x : w2.x);
            w.y = blk == 0 ? w0.y : (blk == 1 ? w1.y : w2.y);
            w.z = blk == 0 ? w0.z : (blk == 1 ? w1.z : w2.z);
            w.w = blk == 0 ? w0.w : (blk == 1 ? w1.w : w2.w);
            e16[k] = sr_lane(w, e & 7);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) u[j] = e16[2 * j] | (e16[2 * j + 1] << 16);
    }
}

__device__ __forceinline__ void sr_draws16(uint64_t seed, uint64_t step, uint64_t idx0, uint32_t (&u)[8])
{
    sr_draws16_at(seed, step, idx0 >> 3, (int)(idx0 & 7u), u);
}

// Same for idx0 = base + lane_off with base the same in every lane and
// lane_off a multiple of 8: the counter is (base >> 3) + (lane_off >> 3), so
// no per-lane 64-bit index is formed.
__device__ __forceinline__ void sr_draws16(uint64_t seed, uint64_t step, uint64_t base, uint32_t lane_off,
                                           uint32_t (&u)[8])
{
    sr_draws16_at(seed, step, (base >> 3) + (lane_off >> 3), (int)(base & 7u), u);
}

// ---------------------------------------------------------------- buffer resources
// Raw buffer descriptors: a lane whose byte offset is at or beyond the
// descriptor's record count reads zeros and its stores are dropped by the
// hardware, so masked lanes need no branch.  Kernels keep every global access
// inside a loop on buffer instructions with such offsets: with no branches
// around memory instructions the compiler's wait counts stay exact, and a
// wait for the next tile's loads does not also wait for the stores issued
// after them.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
constexpr uint32_t kRecords = 0x7FFFFFFFu;   // every in-range offset is below 2^31
constexpr uint32_t kOff = 0x80000000u;       // offset of a masked lane

// Descriptor over [p, p + 2^31): NULL gives an empty one (every access dropped).
__device__ __forceinline__ rsrc_t make_rsrc(const void* p)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, p ? kRecords : 0u, 0x00020000);
}

// Cache policy of the streaming accesses.  Every source byte is read once, and
// non-temporal loads (the "nt" bit) raise streaming bandwidth on MI355X.  The
// tile kernel's code and scale stores are partial-line runs that the L2 must
// merge, and its residual is read and rewritten in place; both keep the
// default policy (measured: non-temporal there costs 1.6x-2x).
constexpr int kNT = 2;

template <int POLICY = kNT>
__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t off)
{
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POLICY);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ float buf_load_f32(rsrc_t r, uint32_t off)
{
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

template <int POLICY = 0>
__device__ __forceinline__ void buf_store16(rsrc_t r, uint32_t off, uint4 v)
{
    const u32x4_t w = {v.x, v.y, v.z, v.w};
    __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, POLICY);
}

template <int POLICY = 0>
__device__ __forceinline__ void buf_store8(rsrc_t r, uint32_t off, uint2 v)
{
    const u32x2_t w = {v.x, v.y};
    __builtin_amdgcn_raw_buffer_store_b64(w, r, off, 0, POLICY);
}

__device__ __forceinline__ void buf_store_u32(rsrc_t r, uint32_t off, uint32_t v)
{
    __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0);
}

__device__ __forceinline__ void buf_store_u8(rsrc_t r, uint32_t off, uint32_t v)
{
    __builtin_amdgcn_raw_buffer_store_b8((unsigned char)v, r, off, 0, 0);
}

// Non-temporal 16-byte global load / store and narrower stores (plain
// pointers).
__device__ __forceinline__ uint4 ld_nt16(const void* p)
{
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ void st_nt16(void* p, uint4 v)
{
    const u32x4_t w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}

__device__ __forceinline__ void st_nt64(void* p, uint2 v)
{
    const u32x2_t w = {v.x, v.y};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2_t*>(p));
}


__device__ __forceinline__ void st_nt32(void* p, uint32_t v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p));
}

__device__ __forceinline__ void st_nt8(void* p, uint32_t v)
{
    __builtin_nontemporal_store((unsigned char)v, reinterpret_cast<unsigned char*>(p));
}

// Wait until every outstanding vector memory operation of this wave has
// completed (s_waitcnt vmcnt(0); expcnt and lgkmcnt left alone).
__device__ __forceinline__ void wait_vmem_all()
{
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

// ---------------------------------------------------------------- LDS-only barrier
// Workgroup barrier whose fences cover LDS only: it orders the workgroup's LDS
// writes before the barrier against LDS reads after it, but does not wait for
// this wave's outstanding global loads and stores, so prefetched loads stay in
// flight across it.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------- packed 16-bit max
typedef unsigned short fp4q_u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b)
{
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(fp4q_u16x2, a),
                                                                  __builtin_bit_cast(fp4q_u16x2, b)));
}

// Largest |x| bit pattern among 2*N packed bf16 (an order-preserving key for
// the magnitudes; any value >= 0x7F80 means an inf or NaN is present).
template <int N>
__device__ __forceinline__ uint32_t bf16_absmax_bits(const uint32_t (&w)[N])
{
    uint32_t m = w[0] & 0x7FFF7FFFu;
#pragma unroll
    for (int k = 1; k < N; ++k) m = pk_max_u16(m, w[k] & 0x7FFF7FFFu);
    const uint32_t lo = m & 0xFFFFu, hi = m >> 16;
    return lo > hi ? lo : hi;
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

// ---------------------------------------------------------------- cross-lane max (DPP)
// Unsigned max with a DPP-permuted copy; lanes outside the row/bank mask see 0,
// which is neutral for the non-negative values reduced here (magnitudes, or
// float bit patterns of magnitudes, which order like the floats).
template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ uint32_t max_dpp(uint32_t v)
{
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWMASK, 0xF, false);
    return v > o ? v : o;
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppBcast15 = 0x142;
constexpr int kDppBcast31 = 0x143;
constexpr int kDppRowRor4 = 0x124;    // rotate right by 4 within each row of 16 lanes
constexpr int kDppRowRor8 = 0x128;    // rotate right by 8 within each row of 16 lanes

// Max over aligned groups of 2 or 4 consecutive lanes (width 1, 2 or 4).
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v, int width)
{
    if (width > 1) v = max_dpp<kDppXor1>(v);
    if (width > 2) v = max_dpp<kDppXor2>(v);
    return v;
}

// Max over the whole wave64, returned uniformly.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max_dpp<kDppXor1>(v);
    v = max_dpp<kDppXor2>(v);
    v = max_dpp<kDppHalfMirror>(v);
    v = max_dpp<kDppMirror>(v);             // every lane holds its row-of-16 max
    v = max_dpp<kDppBcast15, 0xA>(v);      // rows 1, 3 take in rows 0, 2
    v = max_dpp<kDppBcast31, 0xC>(v);      // rows 2, 3 take in rows 0-1
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ float quad_max(float v, int width)
{
    return __uint_as_float(quad_max_u32(__float_as_uint(v), width));
}

// ---------------------------------------------------------------- legacy cross-lane max
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
