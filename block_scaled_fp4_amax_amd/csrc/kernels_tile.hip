// kernels_tile.hip -- 64 x 64 tile kernel for gfx950: fused cast-transpose
// (rowwise and columnwise NVFP4 / AMD-FP4 buffers from one read of the
// source), the 2D outer-block mode, and its grouped (per-expert) form.
//
// "Block-Scaled FP8 and FP4 Weight Quantization", sections 2-4: a fused
// cast-transpose scans the high-precision source once and writes both the
// rowwise buffer and the columnwise buffer (the rowwise layout of W^T); with
// 1D scaling the columnwise direction is its own quantisation of the source
// (blocks run down the columns), not a transpose of the rowwise result.
// "NVFP4 / AMD-FP4 outer-block (two-level) scaling", Technical design and
// Implementation: a 2D outer scale is axis-invariant, computed once per tile
// and used by both directions; 1D outer groups follow the direction
// (1 x obs along rows, obs x 1 along columns); grouped MoE quantisation keeps
// one outer grid per expert.
//
// Per workgroup (256 lanes, 4 waves) one 64 x 64 source tile:
//   row phase  lane (r = t/4, s = t%4) owns the 16-element row block
//              [r, 16s .. 16s+15]: two 16-byte loads, (residual add),
//              outer scale (2D: block-wide max; 1D: max over the obs/16 lanes
//              of the row group), normalise, quantise, store 8 bytes of codes
//              and one scale byte; (qdq output, residual update).
//   LDS        the tile's values (normalised for 2D / tensorwise / none, raw
//              for 1D) and SR draws, so each element keeps one draw in both
//              directions.
//   col phase  lane (c = t/4, q = t%4) owns the column block [16q .. 16q+15, c]:
//              (1D: column outer scale over obs/16 lanes), quantise, store
//              8 bytes of columnwise codes; the 4 lanes of a column write its
//              32 contiguous bytes.
// Tiles are taken in row-major order, split into 8 contiguous slices, one per
// XCD (workgroup ids are dealt round-robin to the XCDs), so the partial cache
// lines that neighbouring tiles write meet in the same L2.
#include "fp4q_device.h"
#include "launch.h"

namespace fp4q {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;

__device__ __forceinline__ void sr_draws16_t(uint64_t seed, uint64_t step, uint64_t idx0, uint32_t (&u)[16])
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

template <int BIAS, bool SR>
__device__ __forceinline__ uint32_t quant16(const float (&vn)[16], const uint32_t (&u)[16], uint2& packed,
                                            float (&p)[16])
{
    float b = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) b = fmaxf(b, __builtin_fabsf(vn[k]));
    const uint32_t cs = scale_encode<BIAS>(b / 6.0f);
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
        const float pm = e2m1_value(m) * d;
        p[k] = sgn ? -pm : pm;
    }
    packed = make_uint2(lo, hi);
    return cs;
}

__device__ __forceinline__ float lanes_max(float v, int width)
{
    // max over aligned groups of `width` (1, 2 or 4) consecutive lanes
    if (width > 1) v = fmaxf(v, __shfl_xor(v, 1, 64));
    if (width > 2) v = fmaxf(v, __shfl_xor(v, 2, 64));
    return v;
}

template <int BIAS, int OUTER, bool SR, bool COLS>
__global__ __launch_bounds__(kThreads) void k_tile(TileArgs a)
{
    __shared__ float lds_v[kTile][kTile + 1];
    __shared__ uint16_t lds_u[SR ? kTile : 1][SR ? kTile + 2 : 1];
    __shared__ float red[kThreads / 64];

    const int bid = (int)blockIdx.x;
    const int tile = (bid & 7) * a.per_xcd + (bid >> 3);
    if (tile >= a.total_tiles) return;   // uniform per workgroup
    int g = 0;
    while (g + 1 < a.ngroups && a.tile0[g + 1] <= tile) ++g;
    const int lt = tile - a.tile0[g];
    const int ti = lt / a.tiles_c, tj = lt - ti * a.tiles_c;
    const int64_t cols = a.cols;
    const int64_t Rg = (int64_t)(a.row0[g + 1] - a.row0[g]);
    const int64_t lrow0 = (int64_t)ti * kTile;          // first tile row inside the group
    const int64_t grow0 = (int64_t)a.row0[g] + lrow0;  // ... in the stacked tensor
    const int64_t c0 = (int64_t)tj * kTile;
    const int rows_valid = (int)min((int64_t)kTile, Rg - lrow0);
    const int cols_valid = (int)min((int64_t)kTile, cols - c0);
    const float den = ScaleFmt<BIAS>::outer_den();

    const int tid = (int)threadIdx.x;
    const int r = tid >> 2, sg = tid & 3;
    const bool act = (r < rows_valid) && (16 * sg < cols_valid);
    const int64_t i_g = grow0 + r;
    const int64_t e0 = i_g * cols + c0 + 16 * sg;   // element offset in the stacked row-major tensor

    // ---------------- row phase
    float v[16];
    float z[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) { v[k] = 0.0f; z[k] = 0.0f; }
    if (act) {
        const uint16_t* px = a.x + i_g * a.ld + c0 + 16 * sg;
        const uint4 w0 = *(const uint4*)px;
        const uint4 w1 = *(const uint4*)(px + 8);
        const uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) { v[2 * k] = bf16_lo(w[k]); v[2 * k + 1] = bf16_hi(w[k]); }
        if (a.residual) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 f = *(const float4*)(a.residual + e0 + 4 * q);
                z[4 * q] = f.x; z[4 * q + 1] = f.y; z[4 * q + 2] = f.z; z[4 * q + 3] = f.w;
            }
#pragma unroll
            for (int k = 0; k < 16; ++k) v[k] = v[k] + z[k];
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = sanitize(v[k]);
    }
    uint32_t u[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) u[k] = 0;
    if (SR && act) sr_draws16_t(a.seed, a.step, a.index_base + (uint64_t)e0, u);

    float am = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) am = fmaxf(am, __builtin_fabsf(v[k]));

    float s_row = 1.0f;
    if (OUTER == kOuterTensor) {
        s_row = *a.tensor_scale;
    } else if (OUTER == kOuter2D) {
        const int64_t oidx = ((int64_t)a.row0[g] / kTile) * (cols / kTile) + (int64_t)ti * (cols / kTile) + tj;
        if (a.outer_given) {
            s_row = a.row_outer[oidx];
        } else {
            float m = group_max<64>(am);
            if ((tid & 63) == 0) red[tid >> 6] = m;
            __syncthreads();
            m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
            s_row = m / den;
            if (tid == 0 && a.row_outer) a.row_outer[oidx] = s_row;
        }
    } else if (OUTER == kOuter1D) {
        const int64_t ogr = i_g * (cols / (16 * a.obs16)) + (c0 + 16 * sg) / (16 * a.obs16);
        if (a.outer_given) {
            s_row = act ? a.row_outer[ogr] : 1.0f;
        } else {
            s_row = lanes_max(am, a.obs16) / den;
            if (act && a.row_outer && (sg % a.obs16) == 0) a.row_outer[ogr] = s_row;
        }
    }

    float vn[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        if (OUTER == kOuterNone) vn[k] = v[k];
        else vn[k] = s_row == 0.0f ? __builtin_copysignf(0.0f, v[k]) : v[k] / s_row;
    }
    if (act) {
        uint2 packed;
        float p[16];
        const uint32_t cs = quant16<BIAS, SR>(vn, u, packed, p);
        if (a.row_codes) *(uint2*)(a.row_codes + e0 / 2) = packed;
        if (a.row_scales) a.row_scales[e0 / 16] = (uint8_t)cs;
        if (a.y || a.residual) {
            float w[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) w[k] = (OUTER == kOuterNone) ? p[k] : p[k] * s_row;
            if (a.y) {
                uint32_t o[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) o[k] = f32_to_bf16(w[2 * k]) | (f32_to_bf16(w[2 * k + 1]) << 16);
                *(uint4*)(a.y + e0) = make_uint4(o[0], o[1], o[2], o[3]);
                *(uint4*)(a.y + e0 + 8) = make_uint4(o[4], o[5], o[6], o[7]);
            }
            if (a.residual) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *(float4*)(a.residual + e0 + 4 * q) =
                        make_float4(v[4 * q] - w[4 * q], v[4 * q + 1] - w[4 * q + 1], v[4 * q + 2] - w[4 * q + 2],
                                    v[4 * q + 3] - w[4 * q + 3]);
            }
        }
    }
    if (!COLS) return;

    // ---------------- stage through LDS
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        lds_v[r][16 * sg + k] = (OUTER == kOuter1D) ? v[k] : vn[k];
        if (SR) lds_u[r][16 * sg + k] = (uint16_t)u[k];
    }
    __syncthreads();

    // ---------------- column phase
    const int cc = tid >> 2, rs = tid & 3;
    const bool actc = (cc < cols_valid) && (16 * rs < rows_valid);
    float cv[16];
    uint32_t cu[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        cv[k] = lds_v[16 * rs + k][cc];
        cu[k] = SR ? (uint32_t)lds_u[16 * rs + k][cc] : 0u;
    }
    if (OUTER == kOuter1D) {
        const int64_t colbase = (int64_t)a.row0[g] * cols / (16 * a.obs16);   // this group's col outer array
        const int64_t ogc = colbase + (c0 + cc) * (Rg / (16 * a.obs16)) + (lrow0 + 16 * rs) / (16 * a.obs16);
        float s_col;
        if (a.outer_given) {
            s_col = actc ? a.col_outer[ogc] : 1.0f;
        } else {
            float m = 0.0f;
#pragma unroll
            for (int k = 0; k < 16; ++k) m = fmaxf(m, __builtin_fabsf(cv[k]));
            s_col = lanes_max(m, a.obs16) / den;
            if (actc && a.col_outer && (rs % a.obs16) == 0) a.col_outer[ogc] = s_col;
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) cv[k] = s_col == 0.0f ? __builtin_copysignf(0.0f, cv[k]) : cv[k] / s_col;
    }
    if (actc) {
        uint2 packed;
        float p[16];
        const uint32_t cs = quant16<BIAS, SR>(cv, cu, packed, p);
        const int64_t colrow = c0 + cc;                       // row of the columnwise buffer
        const int64_t gbase = (int64_t)a.row0[g] * cols;      // elements before this group
        const int64_t ce0 = gbase + colrow * Rg + lrow0 + 16 * rs;
        *(uint2*)(a.col_codes + ce0 / 2) = packed;
        a.col_scales[ce0 / 16] = (uint8_t)cs;
    }
}

}  // namespace

hipError_t launch_tiles(int bias, int outer_kind, bool sr, const TileArgs& a, hipStream_t s)
{
    const dim3 grid(8 * a.per_xcd);
    const bool cols = (a.col_codes != nullptr);
#define FP4Q_T(B, O, S, C) hipLaunchKernelGGL((k_tile<B, O, S, C>), grid, dim3(kThreads), 0, s, a)
#define FP4Q_T_C(B, O, S)                      \
    do {                                       \
        if (cols) FP4Q_T(B, O, S, true);       \
        else FP4Q_T(B, O, S, false);           \
    } while (0)
#define FP4Q_T_S(B, O)                         \
    do {                                       \
        if (sr) FP4Q_T_C(B, O, true);          \
        else FP4Q_T_C(B, O, false);            \
    } while (0)
#define FP4Q_T_O(B)                                            \
    do {                                                       \
        if (outer_kind == kOuterNone) FP4Q_T_S(B, kOuterNone); \
        else if (outer_kind == kOuterTensor) FP4Q_T_S(B, kOuterTensor); \
        else if (outer_kind == kOuter1D) FP4Q_T_S(B, kOuter1D); \
        else FP4Q_T_S(B, kOuter2D);                            \
    } while (0)
    if (bias == 7) FP4Q_T_O(7);
    else FP4Q_T_O(15);
#undef FP4Q_T_O
#undef FP4Q_T_S
#undef FP4Q_T_C
#undef FP4Q_T
    return hipGetLastError();
}

}  // namespace fp4q
