// kernels_nv.hip -- rowwise NVFP4 / AMD-FP4 quantisation (inner scales only,
// tensorwise FP32 scale, or 1D 1 x obs outer-block FP32 scales), the
// tensorwise amax passes, and the NVFP4 / AMD-FP4 dequantiser, for gfx950.
//
// Numerics ("fp4-train" README, Method; "NVFP4 / AMD-FP4 outer-block
// (two-level) scaling for FP4 training", Background, Technical design,
// Implementation), every step one binary32 operation rounded to nearest:
//   v   = x (+ residual)                    error feedback adds the carried residual
//   s_o = A / (scale_max * 6)               A = amax of the outer group, kept in FP32
//   v_n = v / s_o                           (s_o == 0: the group is +-0)
//   d   = dec(enc(max|v_n| / 6))            per-16 block, E4M3 or UE5M3, RNE, satfinite
//   t   = |v_n| / d                         (d == 0: t = 0)
//   m   = RNE(t) or SR(t, u16)              E2M1, sign bit from v_n
//   w   = G[m] * d * s_o                    dequantised value (G[m]*d exact)
//   residual' = v - (+-w)
//
// Work decomposition: one lane owns one 16-element inner block (two 16-byte
// loads); the obs/16 lanes of a 1D outer group are neighbours and combine
// their maxima with cross-lane steps.
#include "fp4q_device.h"
#include "launch.h"

namespace fp4q {

namespace {

constexpr int kThreads = 256;

// 16 SR variates for elements idx0 .. idx0+15 (idx0 = global index of the
// block's first element); draws 2 Philox blocks, or 3 when idx0 % 8 != 0.
__device__ __forceinline__ void sr_draws16(uint64_t seed, uint64_t step, uint64_t idx0, uint32_t (&u)[16])
{
    const uint64_t b0 = idx0 >> 3;
    const int off = (int)(idx0 & 7u);
    const u32x4 w0 = sr_words(seed, step, b0);
    const u32x4 w1 = sr_words(seed, step, b0 + 1);
    u32x4 w2 = w1;
    if (off != 0) w2 = sr_words(seed, step, b0 + 2);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int e = off + k;
        const u32x4& w = (e >> 3) == 0 ? w0 : ((e >> 3) == 1 ? w1 : w2);
        u[k] = sr_lane(w, e & 7);
    }
}

__device__ __forceinline__ void load16_bf16(const uint16_t* p, float (&v)[16])
{
    const uint4 a = *(const uint4*)p;
    const uint4 b = *(const uint4*)(p + 8);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) { v[2 * k] = bf16_lo(w[k]); v[2 * k + 1] = bf16_hi(w[k]); }
}

__device__ __forceinline__ void load16_f32(const float* p, float (&z)[16])
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float4 f = *(const float4*)(p + 4 * q);
        z[4 * q] = f.x; z[4 * q + 1] = f.y; z[4 * q + 2] = f.z; z[4 * q + 3] = f.w;
    }
}

__device__ __forceinline__ void store16_f32(float* p, const float (&z)[16])
{
#pragma unroll
    for (int q = 0; q < 4; ++q) *(float4*)(p + 4 * q) = make_float4(z[4 * q], z[4 * q + 1], z[4 * q + 2], z[4 * q + 3]);
}

// Quantise one 16-element block of normalised values; returns the scale code,
// writes the packed codes and (optionally) the signed inner-dequantised values
// p = +-G[m] * d.
template <int BIAS, bool SR>
__device__ __forceinline__ uint32_t quant_block16(const float (&vn)[16], const uint32_t (&u)[16], uint2& packed,
                                                  float (&p)[16])
{
    float b = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) b = fmaxf(b, __builtin_fabsf(vn[k]));
    const float ys = b / 6.0f;
    const uint32_t cs = scale_encode<BIAS>(ys);
    const float d = scale_decode<BIAS>(cs);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const float t = d == 0.0f ? 0.0f : __builtin_fabsf(vn[k]) / d;
        const uint32_t m = SR ? e2m1_sr(t, u[k]) : e2m1_rne(t);
        const uint32_t sgn = __float_as_uint(vn[k]) >> 31;
        const uint32_t code = m | (sgn << 3);
        if (k < 8) lo |= code << (4 * k);
        else hi |= code << (4 * (k - 8));
        const float pm = e2m1_value(m) * d;   // exact
        p[k] = sgn ? -pm : pm;
    }
    packed = make_uint2(lo, hi);
    return cs;
}

template <int W>
__device__ __forceinline__ float runtime_group_max(float v, int width)
{
#pragma unroll
    for (int m = 1; m < W; m <<= 1)
        if (m < width) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}

template <int BIAS, int OUTER, bool SR>
__global__ __launch_bounds__(kThreads) void k_nv_rows(RowArgs a, uint32_t nblocks, uint32_t bpr)
{
    const uint32_t b = blockIdx.x * kThreads + threadIdx.x;   // inner block id
    // lanes of one 1D outer group are consecutive and bpr % obs16 == 0, so a
    // group is entirely inside or outside the tensor
    if (b >= nblocks) return;
    const uint32_t i = b / bpr;
    const uint32_t jb = b - i * bpr;
    const int64_t j0 = (int64_t)jb * 16;
    const int64_t e0 = (int64_t)i * a.cols + j0;   // element offset in contiguous outputs

    float v[16];
    load16_bf16(a.x + (int64_t)i * a.ld + j0, v);
    float z[16];
    if (a.residual) {
        load16_f32(a.residual + e0, z);
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = v[k] + z[k];
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = sanitize(v[k]);

    uint32_t u[16];
    if (SR) sr_draws16(a.seed, a.step, a.index_base + (uint64_t)e0, u);

    float s_o = 1.0f;
    if (OUTER == kOuterTensor) {
        s_o = *a.tensor_scale;
    } else if (OUTER == kOuter1D) {
        const int64_t og = (int64_t)i * (a.cols / (16 * a.obs16)) + jb / (uint32_t)a.obs16;
        if (a.outer_given) {
            s_o = a.outer[og];
        } else {
            float am = 0.0f;
#pragma unroll
            for (int k = 0; k < 16; ++k) am = fmaxf(am, __builtin_fabsf(v[k]));
            am = runtime_group_max<8>(am, a.obs16);
            s_o = am / ScaleFmt<BIAS>::outer_den();
            if (a.outer && jb % (uint32_t)a.obs16 == 0) a.outer[og] = s_o;
        }
    }
    float vn[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        if (OUTER == kOuterNone) vn[k] = v[k];
        else vn[k] = s_o == 0.0f ? __builtin_copysignf(0.0f, v[k]) : v[k] / s_o;
    }
    uint2 packed;
    float p[16];
    const uint32_t cs = quant_block16<BIAS, SR>(vn, u, packed, p);
    if (a.codes) *(uint2*)(a.codes + e0 / 2) = packed;
    if (a.scales) a.scales[(int64_t)i * bpr + jb] = (uint8_t)cs;
    if (a.y || a.residual) {
        float w[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) w[k] = (OUTER == kOuterNone) ? p[k] : p[k] * s_o;
        if (a.y) {
            uint32_t o[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) o[k] = f32_to_bf16(w[2 * k]) | (f32_to_bf16(w[2 * k + 1]) << 16);
            *(uint4*)(a.y + e0) = make_uint4(o[0], o[1], o[2], o[3]);
            *(uint4*)(a.y + e0 + 8) = make_uint4(o[4], o[5], o[6], o[7]);
        }
        if (a.residual) {
#pragma unroll
            for (int k = 0; k < 16; ++k) z[k] = v[k] - w[k];
            store16_f32(a.residual + e0, z);
        }
    }
}

// Tensorwise pass 1: per-workgroup maxima of |sanitise(x (+ residual))|.
__global__ __launch_bounds__(kThreads) void k_amax_partial(const uint16_t* __restrict__ x, const float* __restrict__ res,
                                                           int64_t cols, int64_t ld, uint32_t nblocks, uint32_t bpr,
                                                           float* __restrict__ partials)
{
    float am = 0.0f;
    for (uint32_t b = blockIdx.x * kThreads + threadIdx.x; b < nblocks; b += gridDim.x * kThreads) {
        const uint32_t i = b / bpr;
        const int64_t j0 = (int64_t)(b - i * bpr) * 16;
        float v[16];
        load16_bf16(x + (int64_t)i * ld + j0, v);
        if (res) {
            float z[16];
            load16_f32(res + (int64_t)i * cols + j0, z);
#pragma unroll
            for (int k = 0; k < 16; ++k) v[k] = v[k] + z[k];
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) am = fmaxf(am, __builtin_fabsf(sanitize(v[k])));
    }
    am = group_max<64>(am);
    __shared__ float wmax[kThreads / 64];
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = am;
    __syncthreads();
    if (threadIdx.x == 0) {
        float m = wmax[0];
        for (int w = 1; w < kThreads / 64; ++w) m = fmaxf(m, wmax[w]);
        partials[blockIdx.x] = m;
    }
}

// Tensorwise pass 2: s_g = RN(max(partials) / (scale_max * 6)).
template <int BIAS>
__global__ __launch_bounds__(kThreads) void k_tensor_scale(const float* __restrict__ partials, int n,
                                                           float* __restrict__ scale_out, float* __restrict__ user_outer)
{
    float m = 0.0f;
    for (int k = threadIdx.x; k < n; k += kThreads) m = fmaxf(m, partials[k]);
    m = group_max<64>(m);
    __shared__ float wmax[kThreads / 64];
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float a = wmax[0];
        for (int w = 1; w < kThreads / 64; ++w) a = fmaxf(a, wmax[w]);
        const float s = a / ScaleFmt<BIAS>::outer_den();
        *scale_out = s;
        if (user_outer) *user_outer = s;
    }
}

// Dequantise one 16-code block: y = bf16(+-G[m] * d [* s_o]).
template <int BIAS>
__global__ __launch_bounds__(kThreads) void k_nv_dequant(const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales,
                                                         const float* __restrict__ outer, int outer_kind,
                                                         int outer_t, int obs, uint32_t nblocks, uint32_t bpr,
                                                         int64_t rows, int64_t cols, uint16_t* __restrict__ y)
{
    const uint32_t b = blockIdx.x * kThreads + threadIdx.x;
    if (b >= nblocks) return;
    const uint32_t i = b / bpr;
    const int64_t j0 = (int64_t)(b - i * bpr) * 16;
    const int64_t e0 = (int64_t)i * cols + j0;
    const uint2 cw = *(const uint2*)(codes + e0 / 2);
    const float d = scale_decode<BIAS>(scales[b]);
    float s_o = 1.0f;
    if (outer_kind == kOuterTensor) s_o = outer[0];
    else if (outer_kind == kOuter1D) s_o = outer[(int64_t)i * (cols / obs) + j0 / obs];
    else if (outer_kind == kOuter2D)
        s_o = outer_t ? outer[(j0 / obs) * (rows / obs) + i / obs] : outer[(int64_t)(i / obs) * (cols / obs) + j0 / obs];
    uint32_t o[8];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const uint32_t code = ((k < 8 ? cw.x : cw.y) >> (4 * (k & 7))) & 0xFu;
        float w = e2m1_value(code & 7u) * d;
        if (outer_kind != kOuterNone) w = w * s_o;
        if (code & 8u) w = -w;
        const uint32_t h = f32_to_bf16(w);
        if (k & 1) o[k >> 1] |= h << 16;
        else o[k >> 1] = h;
    }
    *(uint4*)(y + e0) = make_uint4(o[0], o[1], o[2], o[3]);
    *(uint4*)(y + e0 + 8) = make_uint4(o[4], o[5], o[6], o[7]);
}

}  // namespace

hipError_t launch_rows(int bias, int outer_kind, bool sr, const RowArgs& a, hipStream_t s)
{
    const uint32_t bpr = (uint32_t)(a.cols / 16);
    const uint32_t nblocks = (uint32_t)(a.rows * bpr);
    const uint32_t grid = (nblocks + kThreads - 1) / kThreads;
#define FP4Q_ROWS(B, O, S) hipLaunchKernelGGL((k_nv_rows<B, O, S>), dim3(grid), dim3(kThreads), 0, s, a, nblocks, bpr)
#define FP4Q_ROWS_O(B, S)                                           \
    do {                                                            \
        if (outer_kind == kOuterNone) FP4Q_ROWS(B, kOuterNone, S);   \
        else if (outer_kind == kOuterTensor) FP4Q_ROWS(B, kOuterTensor, S); \
        else FP4Q_ROWS(B, kOuter1D, S);                             \
    } while (0)
    if (bias == 7) { if (sr) FP4Q_ROWS_O(7, true); else FP4Q_ROWS_O(7, false); }
    else { if (sr) FP4Q_ROWS_O(15, true); else FP4Q_ROWS_O(15, false); }
#undef FP4Q_ROWS_O
#undef FP4Q_ROWS
    return hipGetLastError();
}

hipError_t launch_amax(int bias, const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, const float* residual,
                       float* partials, int npartials, float* scale_out, float* user_outer, hipStream_t s)
{
    const uint32_t bpr = (uint32_t)(cols / 16);
    const uint32_t nblocks = (uint32_t)(rows * bpr);
    uint32_t grid = (nblocks + kThreads - 1) / kThreads;
    if (grid > (uint32_t)npartials) grid = (uint32_t)npartials;
    if (grid == 0) grid = 1;
    hipLaunchKernelGGL(k_amax_partial, dim3(grid), dim3(kThreads), 0, s, x, residual, cols, ld, nblocks, bpr, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (bias == 7)
        hipLaunchKernelGGL(k_tensor_scale<7>, dim3(1), dim3(kThreads), 0, s, partials, (int)grid, scale_out, user_outer);
    else
        hipLaunchKernelGGL(k_tensor_scale<15>, dim3(1), dim3(kThreads), 0, s, partials, (int)grid, scale_out, user_outer);
    return hipGetLastError();
}

hipError_t launch_dequant_nv(int bias, int outer_kind, int outer_t, int obs, const uint8_t* codes,
                             const uint8_t* scales, const float* outer, int64_t rows, int64_t cols, uint16_t* y,
                             hipStream_t s)
{
    const uint32_t bpr = (uint32_t)(cols / 16);
    const uint32_t nblocks = (uint32_t)(rows * bpr);
    const uint32_t grid = (nblocks + kThreads - 1) / kThreads;
    if (bias == 7)
        hipLaunchKernelGGL(k_nv_dequant<7>, dim3(grid), dim3(kThreads), 0, s, codes, scales, outer, outer_kind, outer_t,
                           obs, nblocks, bpr, rows, cols, y);
    else
        hipLaunchKernelGGL(k_nv_dequant<15>, dim3(grid), dim3(kThreads), 0, s, codes, scales, outer, outer_kind,
                           outer_t, obs, nblocks, bpr, rows, cols, y);
    return hipGetLastError();
}

}  // namespace fp4q
