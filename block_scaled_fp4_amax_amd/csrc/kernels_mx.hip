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
// with two cross-lane steps.  Each workgroup streams kUnroll * 256 chunks with
// all loads issued before any arithmetic, so a wave keeps kUnroll 16-byte
// requests in flight.  The kernel is HBM-bound; no LDS, no MFMA.
#include "fp4q_device.h"
#include "launch.h"

namespace fp4q {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

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

// Quantise two bf16 halves of one 32-bit word; returns two bf16 results and
// two codes (low nibble = low half).
__device__ __forceinline__ void mx_pair(uint32_t w, float inv_scale, float scale, uint32_t& yw, uint32_t& cw)
{
    float f0 = bf16_lo(w), f1 = bf16_hi(w);
    uint32_t m0 = e2m1_rne(__builtin_fabsf(f0) * inv_scale);
    uint32_t m1 = e2m1_rne(__builtin_fabsf(f1) * inv_scale);
    uint32_t s0 = (w >> 15) & 1u, s1 = w >> 31;
    // G[m] * 2^k is exact in binary32 (<= 2 significant bits, >= 2^-127)
    uint32_t q0 = __float_as_uint(e2m1_value(m0) * scale) >> 16;
    uint32_t q1 = __float_as_uint(e2m1_value(m1) * scale) >> 16;
    yw = (q0 | (s0 << 15)) | ((q1 | (s1 << 15)) << 16);
    cw = (m0 | (s0 << 3)) | ((m1 | (s1 << 3)) << 4);
}

template <bool CONTIG, bool WY, bool WC>
__global__ __launch_bounds__(kThreads) void k_mx_qdq(const uint16_t* __restrict__ x, uint32_t rows, uint32_t cols,
                                                     int64_t ld, uint32_t nchunks, uint16_t* __restrict__ y,
                                                     uint8_t* __restrict__ codes, uint8_t* __restrict__ scales)
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
            in[u] = *(const uint4*)(x + off);
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
        const uint4 w = in[u];
        uint32_t a = 0;
        a = max(a, w.x & 0x7FFFu); a = max(a, (w.x >> 16) & 0x7FFFu);
        a = max(a, w.y & 0x7FFFu); a = max(a, (w.y >> 16) & 0x7FFFu);
        a = max(a, w.z & 0x7FFFu); a = max(a, (w.z >> 16) & 0x7FFFu);
        a = max(a, w.w & 0x7FFFu); a = max(a, (w.w >> 16) & 0x7FFFu);
        a = group_max_u32<4>(a);
        const bool poisoned = a >= 0x7F80u;   // any inf or NaN in the block
        const int k = mx_exponent(a);
        const float inv_scale = __uint_as_float((uint32_t)(127 - k) << 23);
        const float scale = __uint_as_float((uint32_t)(127 + k) << 23);
        uint4 yo;
        uint32_t c0, c1, c2, c3;
        mx_pair(w.x, inv_scale, scale, yo.x, c0);
        mx_pair(w.y, inv_scale, scale, yo.y, c1);
        mx_pair(w.z, inv_scale, scale, yo.z, c2);
        mx_pair(w.w, inv_scale, scale, yo.w, c3);
        uint32_t cw = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
        if (poisoned) {
            yo = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
            cw = 0;
        }
        size_t yoff;
        if (CONTIG) yoff = (size_t)c * 8;
        else { uint32_t r = c / cpr; yoff = (size_t)r * cols + (size_t)(c - r * cpr) * 8; }
        if (WY) *(uint4*)(y + yoff) = yo;
        if (WC) {
            *(uint32_t*)(codes + yoff / 2) = cw;
            if ((c & 3u) == 0) scales[yoff / 32] = poisoned ? 0xFFu : (uint8_t)(k + 127);
        }
    }
}

// Dequantise: y = +-G[m] * 2^(s-127); scale byte 0xFF (NaN) -> 0x7FC0.
__global__ __launch_bounds__(kThreads) void k_mx_dequant(const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales, uint32_t nchunks,
                                                         uint16_t* __restrict__ y)
{
    const uint32_t c = blockIdx.x * kThreads + threadIdx.x;  // chunk of 8 elements
    if (c >= nchunks) return;
    const uint32_t cw = *(const uint32_t*)(codes + (size_t)c * 4);
    const uint32_t sb = scales[c >> 2];
    const float scale = sb == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(sb << 23);  // 2^-127 kept
    uint32_t out[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        uint32_t n0 = (cw >> (8 * p)) & 0xFu, n1 = (cw >> (8 * p + 4)) & 0xFu;
        uint32_t q0 = __float_as_uint(e2m1_value(n0 & 7u) * scale) >> 16;
        uint32_t q1 = __float_as_uint(e2m1_value(n1 & 7u) * scale) >> 16;
        out[p] = (q0 | ((n0 >> 3) << 15)) | ((q1 | ((n1 >> 3) << 15)) << 16);
        if (sb == 0xFFu) out[p] = 0x7FC07FC0u;
    }
    *(uint4*)(y + (size_t)c * 8) = make_uint4(out[0], out[1], out[2], out[3]);
}

}  // namespace

hipError_t launch_mx_qdq(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, uint16_t* y, uint8_t* codes,
                         uint8_t* scales, hipStream_t s)
{
    const uint32_t nchunks = (uint32_t)(rows * (cols / 8));
    const uint32_t grid = (nchunks + kThreads * kUnroll - 1) / (kThreads * kUnroll);
    const bool contig = (ld == cols);
    const bool wy = (y != nullptr), wc = (codes != nullptr);
#define FP4Q_MX(C, Y, W) \
    hipLaunchKernelGGL((k_mx_qdq<C, Y, W>), dim3(grid), dim3(kThreads), 0, s, x, (uint32_t)rows, (uint32_t)cols, ld, \
                       nchunks, y, codes, scales)
    if (contig) {
        if (wy && wc) FP4Q_MX(true, true, true);
        else if (wy) FP4Q_MX(true, true, false);
        else FP4Q_MX(true, false, true);
    } else {
        if (wy && wc) FP4Q_MX(false, true, true);
        else if (wy) FP4Q_MX(false, true, false);
        else FP4Q_MX(false, false, true);
    }
#undef FP4Q_MX
    return hipGetLastError();
}

hipError_t launch_dequant_mx(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols, uint16_t* y,
                             hipStream_t s)
{
    const uint32_t nchunks = (uint32_t)(rows * (cols / 8));
    const uint32_t grid = (nchunks + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(k_mx_dequant, dim3(grid), dim3(kThreads), 0, s, codes, scales, nchunks, y);
    return hipGetLastError();
}

}  // namespace fp4q
