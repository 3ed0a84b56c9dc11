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
#include <cstdlib>
#include <mutex>
#include <vector>

#include "launch.h"
#include "nv_block.h"

namespace fp4q {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;


template <int BIAS, bool SR>
__device__ __forceinline__ uint2 quant16(const float (&vn)[16], const uint32_t (&u)[16], const double* tab,
                                         BlockScale<BIAS>& sc)
{
    sc = block_scale<BIAS>(max_abs16(vn), tab);
    if (SR) return codes16_sr<BIAS>(vn, u, sc);
    return codes16_rne(vn, sc.rd);
}

// Where one tile sits: group, tile row / column, valid extent, and this
// lane's row block.
struct TileCoord {
    int g, ti, tj, rows_valid, cols_valid;
    int64_t Rg, lrow0, i_g, c0, e0;
    bool act;
};

__device__ __forceinline__ TileCoord tile_coord(const TileArgs& a, int tile, int r, int sg)
{
    TileCoord c;
    int g = 0;
    while (g + 1 < a.ngroups && a.tile0[g + 1] <= tile) ++g;
    const int lt = tile - a.tile0[g];
    c.g = g;
    c.ti = lt / a.tiles_c;
    c.tj = lt - c.ti * a.tiles_c;
    c.Rg = (int64_t)(a.row0[g + 1] - a.row0[g]);
    c.lrow0 = (int64_t)c.ti * kTile;
    c.c0 = (int64_t)c.tj * kTile;
    c.rows_valid = (int)min((int64_t)kTile, c.Rg - c.lrow0);
    c.cols_valid = (int)min((int64_t)kTile, a.cols - c.c0);
    c.act = (r < c.rows_valid) && (16 * sg < c.cols_valid);
    c.i_g = (int64_t)a.row0[g] + c.lrow0 + r;
    c.e0 = c.i_g * a.cols + c.c0 + 16 * sg;
    return c;
}

// The lane's raw inputs for one tile: 16 bf16 (two 16-byte loads) and, with
// error feedback, the 16 FP32 residuals.
template <bool EF>
struct TileInput {
    uint4 w0, w1;
    float4 z[EF ? 4 : 1];
};

template <bool EF>
__device__ __forceinline__ void load_tile_input(const TileArgs& a, const TileCoord& c, TileInput<EF>& in)
{
    if (c.act) {
        const uint16_t* px = a.x + c.i_g * a.ld + c.c0 + 16 * (threadIdx.x & 3);
        in.w0 = *(const uint4*)px;
        in.w1 = *(const uint4*)(px + 8);
        if (EF) {
#pragma unroll
            for (int q = 0; q < 4; ++q) in.z[q] = *(const float4*)(a.residual + c.e0 + 4 * q);
        }
    } else {
        in.w0 = make_uint4(0, 0, 0, 0);
        in.w1 = make_uint4(0, 0, 0, 0);
        if (EF) {
#pragma unroll
            for (int q = 0; q < 4; ++q) in.z[q] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
}

// Persistent workgroups: workgroup (xcd = id % 8, slot = id / 8) walks the
// tiles xcd * per_xcd + slot + j * wgs_per_xcd of its XCD's contiguous slice,
// loading tile j+1's inputs before it computes tile j.
// Register budget per lane: 64 VGPRs (8 waves per SIMD) for the plain RTNE
// kernels, 72 (7 waves) for 1D outer groups, 128 (4 waves) with stochastic
// rounding or a residual.
template <int BIAS, int OUTER, bool SR, bool COLS, bool EF>
constexpr int tile_waves_per_simd()
{
    return (SR || EF) ? 4 : (OUTER == kOuter1D ? 7 : 8);
}

template <int BIAS, int OUTER, bool SR, bool COLS, bool EF, bool GIVEN>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(tile_waves_per_simd<BIAS, OUTER, SR, COLS, EF>())))
void k_tile(TileArgs a)
{
    __shared__ float lds_v[kTile][kTile + 1];
    __shared__ uint16_t lds_u[SR ? kTile : 1][SR ? kTile + 2 : 1];
    __shared__ float red[kThreads / 64];
    __shared__ double rtab[16];

    const int tid = (int)threadIdx.x;
    const int r = tid >> 2, sg = tid & 3;
    const int xcd = (int)(blockIdx.x & 7u), slot = (int)(blockIdx.x >> 3);
    const int slice0 = xcd * a.per_xcd;
    const int slice_end = min(slice0 + a.per_xcd, a.total_tiles);
    int tile = slice0 + slot;
    if (tile >= slice_end) return;   // uniform per workgroup
    fill_recip_table(rtab, tid);
    const float den = ScaleFmt<BIAS>::outer_den();
    const int64_t cols = a.cols;

    TileInput<EF> in;
    load_tile_input<EF>(a, tile_coord(a, tile, r, sg), in);

    for (;;) {
        const TileCoord cur = tile_coord(a, tile, r, sg);
        // ---- prefetch the next tile's inputs
        const int next = tile + a.wgs_per_xcd;
        const bool has_next = next < slice_end;
        TileInput<EF> nin = in;
        if (has_next) load_tile_input<EF>(a, tile_coord(a, next, r, sg), nin);

        // ---------------- row phase
        float v[16];
        uint32_t am_bits = 0;    // bit pattern of max |v| over the lane's 16 values
        {
            const uint32_t w[8] = {in.w0.x, in.w0.y, in.w0.z, in.w0.w, in.w1.x, in.w1.y, in.w1.z, in.w1.w};
#pragma unroll
            for (int k = 0; k < 8; ++k) { v[2 * k] = bf16_lo(w[k]); v[2 * k + 1] = bf16_hi(w[k]); }
            if (EF) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    v[4 * q] = v[4 * q] + in.z[q].x;
                    v[4 * q + 1] = v[4 * q + 1] + in.z[q].y;
                    v[4 * q + 2] = v[4 * q + 2] + in.z[q].z;
                    v[4 * q + 3] = v[4 * q + 3] + in.z[q].w;
                }
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const uint32_t b = __float_as_uint(v[k]) & 0x7FFFFFFFu;
                    am_bits = am_bits > b ? am_bits : b;
                }
            } else {
                am_bits = bf16_absmax_bits(w) << 16;
            }
            // NaN / inf anywhere in the lane's 16 values (rare): sanitise them
            if (__builtin_expect(am_bits >= 0x7F800000u, 0)) {
                am_bits = 0;
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    v[k] = sanitize(v[k]);
                    const uint32_t b = __float_as_uint(v[k]) & 0x7FFFFFFFu;
                    am_bits = am_bits > b ? am_bits : b;
                }
            }
        }
        uint32_t u[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) u[k] = 0;
        if (SR && cur.act) sr_draws16(a.seed, a.step, a.index_base + (uint64_t)cur.e0, u);

        float s_row = 1.0f;
        if (OUTER == kOuterTensor) {
            s_row = *a.tensor_scale;
        } else if (OUTER == kOuter2D) {
            const int64_t oidx =
                ((int64_t)a.row0[cur.g] / kTile) * (cols / kTile) + (int64_t)cur.ti * (cols / kTile) + cur.tj;
            if (GIVEN) {
                s_row = a.row_outer[oidx];
            } else {
                const uint32_t m = wave_max_u32(am_bits);
                if ((tid & 63) == 0) red[tid >> 6] = __uint_as_float(m);
                lds_barrier();
                s_row = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])) / den;
                if (tid == 0 && a.row_outer) a.row_outer[oidx] = s_row;
            }
        } else if (OUTER == kOuter1D) {
            const int64_t ogr = cur.i_g * (cols / (16 * a.obs16)) + (cur.c0 + 16 * sg) / (16 * a.obs16);
            if (GIVEN) {
                s_row = cur.act ? a.row_outer[ogr] : 1.0f;
            } else {
                s_row = __uint_as_float(quad_max_u32(am_bits, a.obs16)) / den;
                if (cur.act && a.row_outer && (sg % a.obs16) == 0) a.row_outer[ogr] = s_row;
            }
        }
        lds_barrier();   // reciprocal table filled; previous tile's column reads done

        float vn[16];
        if (OUTER == kOuterNone) {
#pragma unroll
            for (int k = 0; k < 16; ++k) vn[k] = v[k];
        } else {
            normalize16(v, s_row, outer_inv(s_row), vn);
        }
        if (cur.act) {
            BlockScale<BIAS> sc;
            const uint2 packed = quant16<BIAS, SR>(vn, u, rtab, sc);
            if (a.row_codes) *(uint2*)(a.row_codes + cur.e0 / 2) = packed;
            if (a.row_scales) a.row_scales[cur.e0 / 16] = (uint8_t)sc.code;
            if (EF || a.y) {
                float w[16];
                decode16(packed, sc.d, w);
                if (OUTER != kOuterNone) {
#pragma unroll
                    for (int k = 0; k < 16; ++k) w[k] = w[k] * s_row;
                }
                if (a.y) {
                    uint32_t o[8];
#pragma unroll
                    for (int k = 0; k < 8; ++k) o[k] = f32_to_bf16(w[2 * k]) | (f32_to_bf16(w[2 * k + 1]) << 16);
                    *(uint4*)(a.y + cur.e0) = make_uint4(o[0], o[1], o[2], o[3]);
                    *(uint4*)(a.y + cur.e0 + 8) = make_uint4(o[4], o[5], o[6], o[7]);
                }
                if (EF) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *(float4*)(a.residual + cur.e0 + 4 * q) =
                            make_float4(v[4 * q] - w[4 * q], v[4 * q + 1] - w[4 * q + 1],
                                        v[4 * q + 2] - w[4 * q + 2], v[4 * q + 3] - w[4 * q + 3]);
                }
            }
        }
        if (COLS) {
            // ---------------- stage through LDS
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                lds_v[r][16 * sg + k] = (OUTER == kOuter1D) ? v[k] : vn[k];
                if (SR) lds_u[r][16 * sg + k] = (uint16_t)u[k];
            }
            lds_barrier();

            // ---------------- column phase
            const int cc = tid >> 2, rs = tid & 3;
            const bool actc = (cc < cur.cols_valid) && (16 * rs < cur.rows_valid);
            float cv[16];
            uint32_t cu[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                cv[k] = lds_v[16 * rs + k][cc];
                cu[k] = SR ? (uint32_t)lds_u[16 * rs + k][cc] : 0u;
            }
            if (OUTER == kOuter1D) {
                const int64_t colbase = (int64_t)a.row0[cur.g] * cols / (16 * a.obs16);
                const int64_t ogc = colbase + (cur.c0 + cc) * (cur.Rg / (16 * a.obs16)) +
                                    (cur.lrow0 + 16 * rs) / (16 * a.obs16);
                float s_col;
                if (GIVEN) {
                    s_col = actc ? a.col_outer[ogc] : 1.0f;
                } else {
                    s_col = quad_max(max_abs16(cv), a.obs16) / den;
                    if (actc && a.col_outer && (rs % a.obs16) == 0) a.col_outer[ogc] = s_col;
                }
                float cn[16];
                normalize16(cv, s_col, outer_inv(s_col), cn);
#pragma unroll
                for (int k = 0; k < 16; ++k) cv[k] = cn[k];
            }
            if (actc) {
                BlockScale<BIAS> sc;
                const uint2 packed = quant16<BIAS, SR>(cv, cu, rtab, sc);
                const int64_t colrow = cur.c0 + cc;                   // row of the columnwise buffer
                const int64_t gbase = (int64_t)a.row0[cur.g] * cols;  // elements before this group
                const int64_t ce0 = gbase + colrow * cur.Rg + cur.lrow0 + 16 * rs;
                *(uint2*)(a.col_codes + ce0 / 2) = packed;
                a.col_scales[ce0 / 16] = (uint8_t)sc.code;
            }
        }
        if (!has_next) break;
        tile = next;
        in = nin;
    }
}

// Workgroups of `fn` resident per CU, and the CU count, of the current
// device (queried once per device and kernel).
struct Residency {
    int wgs_per_cu;
    int cus;
};

Residency residency(const void* fn)
{
    struct Entry {
        int dev;
        const void* fn;
        Residency r;
    };
    static std::mutex mu;
    static std::vector<Entry> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return {1, 8};
    std::lock_guard<std::mutex> lock(mu);
    for (const Entry& e : cache)
        if (e.dev == dev && e.fn == fn) return e.r;
    Residency r{1, 8};
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kThreads, 0) == hipSuccess && n > 0) r.wgs_per_cu = n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n >= 8) r.cus = n;
    cache.push_back({dev, fn, r});
    return r;
}

// Launch one persistent grid: as many workgroups per XCD as fit at once,
// spread so that every workgroup of a slice takes the same number of tiles
// (to within one).
hipError_t launch_persistent(void (*fn)(TileArgs), TileArgs a, hipStream_t s)
{
    const Residency r = residency(reinterpret_cast<const void*>(fn));
    const int cap = r.wgs_per_cu * (r.cus / 8);
    int w = a.wgs_per_xcd < cap ? a.wgs_per_xcd : cap;
    if (w < 1) w = 1;
    const int rounds = (a.per_xcd + w - 1) / w;
    if (rounds > 1) w = (a.per_xcd + rounds - 1) / rounds;
    a.wgs_per_xcd = w;
    hipLaunchKernelGGL(fn, dim3(8 * w), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_tiles(int bias, int outer_kind, bool sr, const TileArgs& a, hipStream_t s)
{
    const bool cols = (a.col_codes != nullptr);
    const bool ef = (a.residual != nullptr);
    const bool given = a.outer_given != 0;
#define FP4Q_T(B, O, S, C, E, G) return launch_persistent(k_tile<B, O, S, C, E, G>, a, s)
#define FP4Q_T_G(B, O, S, C, E)                 \
    do {                                        \
        if (given) FP4Q_T(B, O, S, C, E, true); \
        else FP4Q_T(B, O, S, C, E, false);      \
    } while (0)
#define FP4Q_T_E(B, O, S, C, G)                 \
    do {                                        \
        if (ef) G(B, O, S, C, true);            \
        else G(B, O, S, C, false);              \
    } while (0)
#define FP4Q_T_NG(B, O, S, C, E) FP4Q_T(B, O, S, C, E, false)
#define FP4Q_T_S(B, O, C, G)                    \
    do {                                        \
        if (sr) FP4Q_T_E(B, O, true, C, G);     \
        else FP4Q_T_E(B, O, false, C, G);       \
    } while (0)
#define FP4Q_T_O(B)                                                               \
    do {                                                                          \
        if (!cols) FP4Q_T_S(B, kOuter2D, false, FP4Q_T_G);                        \
        else if (outer_kind == kOuterNone) FP4Q_T_S(B, kOuterNone, true, FP4Q_T_NG); \
        else if (outer_kind == kOuterTensor) FP4Q_T_S(B, kOuterTensor, true, FP4Q_T_NG); \
        else if (outer_kind == kOuter1D) FP4Q_T_S(B, kOuter1D, true, FP4Q_T_G);  \
        else FP4Q_T_S(B, kOuter2D, true, FP4Q_T_G);                               \
    } while (0)
    if (bias == 7) FP4Q_T_O(7);
    FP4Q_T_O(15);
#undef FP4Q_T_O
#undef FP4Q_T_S
#undef FP4Q_T_NG
#undef FP4Q_T_E
#undef FP4Q_T_G
#undef FP4Q_T
}

}  // namespace fp4q
