// kernels_outer.hip -- FP32 outer scales of 1D outer groups that span two
// 64 x 64 tiles (obs = 128), computed ahead of the tile kernel.
//
// "NVFP4 / AMD-FP4 outer-block (two-level) scaling", Technical design: a 1D
// outer group is 1 x obs along the rows (and obs x 1 down the columns for the
// columnwise buffer), obs any multiple of 16 dividing the reduction
// dimension; its scale is RN(amax / (scale_max * 6)) over the values being
// quantised (x, plus the residual with error feedback, sanitised).  The tile
// kernel works on 64 x 64 tiles one at a time, so a 128-element group's
// maximum is taken here, from one read of each 128 x 128 block, and the tile
// kernel then reads the scales as precomputed ones.
//
// One workgroup (256 lanes) per 128 x 128 block of one group:
//   rows     lane (r = t / 2, h = t % 2) reads row r, columns 64 h .. 64 h + 63
//            (eight 16-byte bf16 loads, sixteen of FP32 residual), the two lanes
//            of a row combine their maxima with one DPP step;
//   columns  lane (c = t / 2, h = t % 2) takes column c over rows 64 h .. 64 h +
//            63 from the block just read (cache-resident), the two lanes of a
//            column combine with one DPP step.
#include "launch.h"
#include "nv_block.h"

namespace fp4q {

namespace {

constexpr int kThreads = 256;
constexpr int kB = 128;    // block edge = obs

// |sanitise(x + r)| bit pattern (r may be absent).
__device__ __forceinline__ uint32_t mag_bits(float x, float r, bool ef)
{
    const float v = ef ? x + r : x;
    return __float_as_uint(sanitize(v)) & 0x7FFFFFFFu;
}

template <int BIAS, bool EF>
__global__ __launch_bounds__(kThreads) void k_outer128(TileArgs a, int32_t blocks_c)
{
    const int tid = (int)threadIdx.x;
    const int cols = (int)a.cols;
    const float den = ScaleFmt<BIAS>::outer_den();
    const int gpr = cols / kB;                                 // row groups per row
    // block -> group: tile0[] counts 128 x 128 blocks here
    const int blk = (int)blockIdx.x;
    int g = 0;
    while (g + 1 < a.ngroups && a.tile0[g + 1] <= blk) ++g;
    const int lb = blk - a.tile0[g];
    const int bi = lb / blocks_c, bj = lb - bi * blocks_c;
    const int r0 = a.row0[g];
    const int Rg = a.row0[g + 1] - r0;
    const int64_t grow0 = (int64_t)r0 + (int64_t)bi * kB;      // first source row of the block
    const int c0 = bj * kB;

    // ---- rows
    {
        const int r = tid >> 1, h = tid & 1;
        const int64_t row = grow0 + r;
        const uint16_t* px = a.x + row * a.ld + c0 + 64 * h;
        const float* pz = EF ? a.residual + row * cols + c0 + 64 * h : nullptr;
        uint32_t m = 0;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint4 w = ld_nt16(px + 8 * q);
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
            float z[8];
            if (EF) {
                const uint4 z0 = *reinterpret_cast<const uint4*>(pz + 8 * q);
                const uint4 z1 = *reinterpret_cast<const uint4*>(pz + 8 * q + 4);
                z[0] = __uint_as_float(z0.x); z[1] = __uint_as_float(z0.y); z[2] = __uint_as_float(z0.z); z[3] = __uint_as_float(z0.w);
                z[4] = __uint_as_float(z1.x); z[5] = __uint_as_float(z1.y); z[6] = __uint_as_float(z1.z); z[7] = __uint_as_float(z1.w);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                m = max(m, mag_bits(bf16_lo(ww[k]), EF ? z[2 * k] : 0.0f, EF));
                m = max(m, mag_bits(bf16_hi(ww[k]), EF ? z[2 * k + 1] : 0.0f, EF));
            }
        }
        m = max_dpp<kDppXor1>(m);
        if (h == 0) a.row_outer[row * gpr + bj] = outer_scale(__uint_as_float(m), den);
    }

    // ---- columns (the block is in the caches now)
    {
        const int c = tid >> 1, h = tid & 1;
        const int64_t col = (int64_t)c0 + c;
        uint32_t m = 0;
#pragma unroll 8
        for (int k = 0; k < 64; ++k) {
            const int64_t row = grow0 + 64 * h + k;
            const float x = __uint_as_float((uint32_t)a.x[row * a.ld + col] << 16);
            const float z = EF ? a.residual[row * cols + col] : 0.0f;
            m = max(m, mag_bits(x, z, EF));
        }
        m = max_dpp<kDppXor1>(m);
        // group g's columnwise scales [cols, Rg / 128], stored after the earlier groups'
        if (h == 0) a.col_outer[(int64_t)r0 * gpr + col * (Rg / kB) + bi] = outer_scale(__uint_as_float(m), den);
    }
}

}  // namespace

hipError_t launch_outer128(int bias, const TileArgs& t, hipStream_t s)
{
    TileArgs a = t;
    const int32_t blocks_c = (int32_t)(a.cols / kB);
    int32_t total = 0;
    for (int g = 0; g < a.ngroups; ++g) {
        a.tile0[g] = total;
        total += ((a.row0[g + 1] - a.row0[g]) / kB) * blocks_c;
    }
    a.tile0[a.ngroups] = total;
    if (total == 0) return hipSuccess;
    const bool ef = a.residual != nullptr;
    if (bias == 7) {
        if (ef) hipLaunchKernelGGL((k_outer128<7, true>), dim3(total), dim3(kThreads), 0, s, a, blocks_c);
        else hipLaunchKernelGGL((k_outer128<7, false>), dim3(total), dim3(kThreads), 0, s, a, blocks_c);
    } else {
        if (ef) hipLaunchKernelGGL((k_outer128<15, true>), dim3(total), dim3(kThreads), 0, s, a, blocks_c);
        else hipLaunchKernelGGL((k_outer128<15, false>), dim3(total), dim3(kThreads), 0, s, a, blocks_c);
    }
    return hipGetLastError();
}

}  // namespace fp4q
