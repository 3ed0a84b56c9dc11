// kernels_mx.hip -- MXFP4 (1x32 UE8M0 power-of-two scale, E2M1 RTNE) fake-quant
// and dequantise for gfx950.
//
// "MXFP4 weight QAT recipes on MXFP8 and FP8 block-scaling hosts", Overview and
// Design: a fused bf16 -> mxfp4 (rowwise 1x32) -> bf16 projection whose output
// is exactly representable in bf16; scale floor 2^-126, cap 2^125, derived
// from the integer bits of the block amax; Correctness: inf/NaN poison the
// whole block, +-0 keep their sign, RTNE midpoints, satfinite at 6.
//
// Work decomposition: one lane owns 8 consecutive bf16 (one 16-byte load),
// four neighbouring lanes own one 32-element block and combine their maxima
// (packed 16-bit integer max of |x| bit patterns) with two DPP steps.  The
// E2M1 encode of x / 2^k and the decode of +-G[m] * 2^k are gfx950's scaled
// FP4 conversions, which match the RTNE / satfinite / signed-zero rules
// exactly for every bf16 input and every k in [-126, 125] (checked
// exhaustively on the device).  One 16-byte chunk per lane, with non-temporal
// loads and stores (one chunk per lane and the non-temporal policy measured
// fastest on MI355X: 6.3 TB/s at 8192 x 8192 against 5.6 TB/s for four
// chunks per lane with default caching).  The kernel is HBM-bound; no LDS,
// no MFMA.
//
// FP32 sources and targets ("MXFP4 weight QAT recipes", Correctness: fake-quant
// on bf16 and fp32, dequantise to bf16 and fp32): the lane's 8 values come from
// two 16-byte loads, the amax and k from their binary32 bits by the same rule,
// and y = +-G[m] 2^k is written as FP32 (exact in either type).  A view whose
// start or row pitch is not 16-byte aligned is read one element per load.
#include "fp4q_device.h"
#include "launch.h"

namespace fp4q {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 1;

// Scale exponent k = ceil(log2(amax / 6)) from the bf16 bits of amax
// (amax = 2^e (1 + f)  ->  k = e - 2 + [f > 1/2]), zero and subnormal amax at
// the floor, then clamped to [-126, 125].
__device__ __forceinline__ int mx_exponent(uint32_t abits)
{
    int e = (int)(abits >> 7);
    int k = e - 129 + (int)((abits & 0x7Fu) > 0x40u);
    k = e == 0 ? -126 : k;
    k = k < -126 ? -126 : k;
    return k > 125 ? 125 : k;
}

// bf16 pair (hi halves of two floats): bytes 2-3 of each
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

template <int Q>
__device__ __forceinline__ uint32_t decode_pair_bf16(uint32_t codes, float scale)
{
    auto f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, scale, Q);   // exact +-G[m] * 2^k
    return pack_bf16x2(f[0], f[1]);
}

// The same scale exponent from the binary32 bits of amax (f > 1/2 is a
// fraction field above 0x400000).
__device__ __forceinline__ int mx_exponent32(uint32_t abits)
{
    int e = (int)(abits >> 23);
    int k = e - 129 + (int)((abits & 0x7FFFFFu) > 0x400000u);
    k = e == 0 ? -126 : k;
    k = k < -126 ? -126 : k;
    return k > 125 ? 125 : k;
}

__device__ __forceinline__ void st_y8_f32(float* p, const float (&f)[8])
{
    st_nt16(p, make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])));
    st_nt16(p + 4, make_uint4(__float_as_uint(f[4]), __float_as_uint(f[5]), __float_as_uint(f[6]), __float_as_uint(f[7])));
}

template <int Q>
__device__ __forceinline__ void decode_pair_f32(uint32_t codes, float scale, float& a, float& b)
{
    auto f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, scale, Q);
    a = f[0];
    b = f[1];
}

// FP32-source fake-quant of one 8-element chunk per lane.  VEC: the source
// chunk is 16-byte aligned (two vector loads), otherwise eight 4-byte loads.
template <bool VEC, bool WY, bool WC>
__device__ __forceinline__ void mx_chunk_f32(const float* __restrict__ xp, bool y_f32, void* __restrict__ y,
                                             size_t yoff, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                             uint32_t c, bool live)
{
    float v[8];
    if (live) {
        if (VEC) {
            const uint4 a = ld_nt16(xp), b = ld_nt16(xp + 4);
            const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = __uint_as_float(w[k]);
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = __builtin_nontemporal_load(xp + k);
        }
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = 0.0f;
    }
    uint32_t am = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) am = max(am, __float_as_uint(v[k]) & 0x7FFFFFFFu);
    am = quad_max_u32(am, 4);                       // block amax, binary32 bits
    if (!live) return;
    const bool poisoned = am >= 0x7F800000u;
    const int k = mx_exponent32(am);
    const float scale = __uint_as_float((uint32_t)(127 + k) << 23);
    uint32_t cw = 0;
    cw = fp4x2_rne_scaled<0>(cw, v[0], v[1], scale);
    cw = fp4x2_rne_scaled<1>(cw, v[2], v[3], scale);
    cw = fp4x2_rne_scaled<2>(cw, v[4], v[5], scale);
    cw = fp4x2_rne_scaled<3>(cw, v[6], v[7], scale);
    if (poisoned) cw = 0;
    if (WY) {
        float f[8];
        decode_pair_f32<0>(cw, scale, f[0], f[1]);
        decode_pair_f32<1>(cw, scale, f[2], f[3]);
        decode_pair_f32<2>(cw, scale, f[4], f[5]);
        decode_pair_f32<3>(cw, scale, f[6], f[7]);
        if (poisoned) {
#pragma unroll
            for (int q = 0; q < 8; ++q) f[q] = __uint_as_float(0x7FC00000u);
        }
        if (y_f32) {
            st_y8_f32(static_cast<float*>(y) + yoff, f);
        } else {
            uint4 yo;
            yo.x = pack_bf16x2(f[0], f[1]);
            yo.y = pack_bf16x2(f[2], f[3]);
            yo.z = pack_bf16x2(f[4], f[5]);
            yo.w = pack_bf16x2(f[6], f[7]);
            st_nt16(static_cast<uint16_t*>(y) + yoff, yo);
        }
    }
    if (WC) {
        st_nt32(codes + yoff / 2, cw);
        if ((c & 3u) == 0) st_nt8(scales + yoff / 32, poisoned ? 0xFFu : (uint32_t)(k + 127));
    }
}

template <bool VEC, bool WY, bool WC>
__global__ __launch_bounds__(kThreads) void k_mx_qdq_f32(const float* __restrict__ x, uint32_t cols, int64_t ld,
                                                         uint32_t nchunks, void* __restrict__ y, int y_f32,
                                                         uint8_t* __restrict__ codes, uint8_t* __restrict__ scales)
{
    const uint32_t cpr = cols >> 3;
    const uint32_t c = blockIdx.x * kThreads + threadIdx.x;
    // the four lanes of a block are consecutive and nchunks % 4 == 0, so they
    // are all inside or all outside the tensor
    const bool live = c < nchunks;
    const uint32_t r = c / cpr;
    const size_t xoff = (size_t)r * (size_t)ld + (size_t)(c - r * cpr) * 8;
    const size_t yoff = (size_t)r * cols + (size_t)(c - r * cpr) * 8;
    mx_chunk_f32<VEC, WY, WC>(x + (live ? xoff : 0), y_f32 != 0, y, yoff, codes, scales, c, live);
}

template <bool CONTIG, bool VEC, bool WY, bool WC>
__global__ __launch_bounds__(kThreads) void k_mx_qdq(const uint16_t* __restrict__ x, uint32_t rows, uint32_t cols,
                                                     int64_t ld, uint32_t nchunks, void* __restrict__ yv,
                                                     int y_f32, uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales)
{
    const uint32_t cpr = cols >> 3;  // 8-element chunks per row
    const uint32_t base = blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
    uint4 in[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        uint32_t c = base + u * kThreads;
        if (c < nchunks) {
            size_t off;
            if (CONTIG) off = (size_t)c * 8;
            else { uint32_t r = c / cpr; off = (size_t)r * (size_t)ld + (size_t)(c - r * cpr) * 8; }
            if (VEC) {
                in[u] = ld_nt16(x + off);
            } else {
                uint32_t h[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) h[k] = __builtin_nontemporal_load(x + off + k);
                in[u] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
            }
        } else {
            in[u] = make_uint4(0, 0, 0, 0);
        }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const uint32_t c = base + u * kThreads;
        // the four lanes of a block are consecutive and nchunks % 4 == 0, so
        // they are all inside or all outside the tensor
        if (c >= nchunks) continue;
        const uint32_t w[4] = {in[u].x, in[u].y, in[u].z, in[u].w};
        const uint32_t a = quad_max_u32(bf16_absmax_bits(w), 4);   // block amax, as bf16 bits
        const bool poisoned = a >= 0x7F80u;                          // any inf or NaN in the block
        const int k = mx_exponent(a);
        const float scale = __uint_as_float((uint32_t)(127 + k) << 23);   // 2^k
        // codes of x / 2^k: hardware RNE onto E2M1, sign kept
        uint32_t cw = 0;
        cw = fp4x2_rne_scaled<0>(cw, bf16_lo(w[0]), bf16_hi(w[0]), scale);
        cw = fp4x2_rne_scaled<1>(cw, bf16_lo(w[1]), bf16_hi(w[1]), scale);
        cw = fp4x2_rne_scaled<2>(cw, bf16_lo(w[2]), bf16_hi(w[2]), scale);
        cw = fp4x2_rne_scaled<3>(cw, bf16_lo(w[3]), bf16_hi(w[3]), scale);
        if (poisoned) cw = 0;
        size_t yoff;
        if (CONTIG) yoff = (size_t)c * 8;
        else { uint32_t r = c / cpr; yoff = (size_t)r * cols + (size_t)(c - r * cpr) * 8; }
        if (WY && y_f32) {
            float f[8];
            decode_pair_f32<0>(cw, scale, f[0], f[1]);
            decode_pair_f32<1>(cw, scale, f[2], f[3]);
            decode_pair_f32<2>(cw, scale, f[4], f[5]);
            decode_pair_f32<3>(cw, scale, f[6], f[7]);
            if (poisoned) {
#pragma unroll
                for (int q = 0; q < 8; ++q) f[q] = __uint_as_float(0x7FC00000u);
            }
            st_y8_f32(static_cast<float*>(yv) + yoff, f);
        } else if (WY) {
            uint4 yo;
            yo.x = decode_pair_bf16<0>(cw, scale);
            yo.y = decode_pair_bf16<1>(cw, scale);
            yo.z = decode_pair_bf16<2>(cw, scale);
            yo.w = decode_pair_bf16<3>(cw, scale);
            if (poisoned) yo = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
            st_nt16(static_cast<uint16_t*>(yv) + yoff, yo);
        }
        if (WC) {
            st_nt32(codes + yoff / 2, cw);
            if ((c & 3u) == 0) st_nt8(scales + yoff / 32, poisoned ? 0xFFu : (uint32_t)(k + 127));
        }
    }
}

// Dequantise: y = +-G[m] * 2^(s-127) (2^-127 for s == 0 kept); scale byte
// 0xFF (NaN) -> the quiet NaN (0x7FC0, or 0x7FC00000 with YF32).
template <bool YF32>
__global__ __launch_bounds__(kThreads) void k_mx_dequant(const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales, uint32_t nchunks,
                                                         void* __restrict__ y)
{
    const uint32_t c = blockIdx.x * kThreads + threadIdx.x;  // chunk of 8 elements
    if (c >= nchunks) return;
    const uint32_t cw = *(const uint32_t*)(codes + (size_t)c * 4);
    const uint32_t sb = scales[c >> 2];
    const float scale = sb == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(sb << 23);
    if (YF32) {
        float f[8];
        decode_pair_f32<0>(cw, scale, f[0], f[1]);
        decode_pair_f32<1>(cw, scale, f[2], f[3]);
        decode_pair_f32<2>(cw, scale, f[4], f[5]);
        decode_pair_f32<3>(cw, scale, f[6], f[7]);
        if (sb == 0xFFu) {
#pragma unroll
            for (int q = 0; q < 8; ++q) f[q] = __uint_as_float(0x7FC00000u);
        }
        st_y8_f32(static_cast<float*>(y) + (size_t)c * 8, f);
        return;
    }
    uint4 yo;
    yo.x = decode_pair_bf16<0>(cw, scale);
    yo.y = decode_pair_bf16<1>(cw, scale);
    yo.z = decode_pair_bf16<2>(cw, scale);
    yo.w = decode_pair_bf16<3>(cw, scale);
    if (sb == 0xFFu) yo = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
    st_nt16(static_cast<uint16_t*>(y) + (size_t)c * 8, yo);
}

}  // namespace

hipError_t launch_mx_qdq(const void* x, bool x_f32, bool x_vec, int64_t rows, int64_t cols, int64_t ld, void* y,
                         bool y_f32, uint8_t* codes, uint8_t* scales, hipStream_t s)
{
    const uint32_t nchunks = (uint32_t)(rows * (cols / 8));
    const uint32_t grid = (nchunks + kThreads * kUnroll - 1) / (kThreads * kUnroll);
    const bool wy = (y != nullptr), wc = (codes != nullptr);
    const int yf = y_f32 ? 1 : 0;
    if (x_f32) {
        const float* xf = static_cast<const float*>(x);
#define FP4Q_MXF(V, Y, W) \
    hipLaunchKernelGGL((k_mx_qdq_f32<V, Y, W>), dim3(grid), dim3(kThreads), 0, s, xf, (uint32_t)cols, ld, nchunks, y, \
                       yf, codes, scales)
#define FP4Q_MXF_V(V)                          \
    do {                                       \
        if (wy && wc) FP4Q_MXF(V, true, true); \
        else if (wy) FP4Q_MXF(V, true, false); \
        else FP4Q_MXF(V, false, true);         \
    } while (0)
        if (x_vec) FP4Q_MXF_V(true);
        else FP4Q_MXF_V(false);
#undef FP4Q_MXF_V
#undef FP4Q_MXF
        return hipGetLastError();
    }
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const bool contig = (ld == cols) && x_vec;
#define FP4Q_MX(C, V, Y, W) \
    hipLaunchKernelGGL((k_mx_qdq<C, V, Y, W>), dim3(grid), dim3(kThreads), 0, s, xb, (uint32_t)rows, (uint32_t)cols, ld, \
                       nchunks, y, yf, codes, scales)
#define FP4Q_MX_CV(C, V)                          \
    do {                                          \
        if (wy && wc) FP4Q_MX(C, V, true, true);  \
        else if (wy) FP4Q_MX(C, V, true, false);  \
        else FP4Q_MX(C, V, false, true);          \
    } while (0)
    if (contig) FP4Q_MX_CV(true, true);
    else if (x_vec) FP4Q_MX_CV(false, true);
    else FP4Q_MX_CV(false, false);
#undef FP4Q_MX_CV
#undef FP4Q_MX
    return hipGetLastError();
}

hipError_t launch_dequant_mx(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols, void* y,
                             bool y_f32, hipStream_t s)
{
    const uint32_t nchunks = (uint32_t)(rows * (cols / 8));
    const uint32_t grid = (nchunks + kThreads - 1) / kThreads;
    if (y_f32) hipLaunchKernelGGL(k_mx_dequant<true>, dim3(grid), dim3(kThreads), 0, s, codes, scales, nchunks, y);
    else hipLaunchKernelGGL(k_mx_dequant<false>, dim3(grid), dim3(kThreads), 0, s, codes, scales, nchunks, y);
    return hipGetLastError();
}

}  // namespace fp4q
