// abi_driver.cpp -- exercises the host side of libfp4q.so (validation, size
// queries, staging plans, status strings) for every entry point, built with
// -fsanitize=address,undefined on the host code by tests/test_sanitizers.py.
// Every call here either fails validation before anything is enqueued or is a
// pure host query, so device pointers are never dereferenced; the driver
// refuses to run where a GPU is visible (it would then be the wrong tool).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/fp4q.h"

static int failures = 0;
#define EXPECT(call, want)                                                                          \
    do {                                                                                            \
        const int got_ = (call);                                                                    \
        if (got_ != (want)) {                                                                       \
            std::fprintf(stderr, "line %d: %s -> %d (%s), want %d\n", __LINE__, #call, got_,        \
                         fp4q_status_str(got_), (int)(want));                                       \
            ++failures;                                                                             \
        }                                                                                           \
    } while (0)

static fp4q_cfg cfg(int format = FP4Q_NVFP4, int two_level = FP4Q_TWO_LEVEL_NONE, int obs = 0, int o2d = 0,
                    int rounding = FP4Q_RNE)
{
    fp4q_cfg c;
    std::memset(&c, 0, sizeof(c));
    c.abi_version = FP4Q_ABI_VERSION;
    c.format = format;
    c.two_level = two_level;
    c.outer_block_size = obs;
    c.outer_2d = o2d;
    c.rounding = rounding;
    return c;
}

int main()
{
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0) {
        std::printf("abi driver: a GPU is visible, skipped (host-only check)\n");
        return 0;
    }
    uint8_t* const F = reinterpret_cast<uint8_t*>(0x10000);   // 16-byte aligned, never dereferenced
    uint8_t* const F4 = reinterpret_cast<uint8_t*>(0x10004);  // 4-byte aligned only
    float* const Ff = reinterpret_cast<float*>(F);
    uint16_t* const Fx = reinterpret_cast<uint16_t*>(F);

    for (int s = -1; s < 12; ++s) {
        const char* t = fp4q_status_str(s);
        if (!t || !*t) ++failures;
    }
    if (fp4q_abi_version() != FP4Q_ABI_VERSION) ++failures;

    // configuration rules
    fp4q_cfg c = cfg();
    c.abi_version = 0;
    EXPECT(fp4_quantize(&c, F, 64, 64, 64, F, F, nullptr, nullptr, nullptr, 0, nullptr), FP4Q_ERR_ABI);
    EXPECT(fp4_quantize(nullptr, F, 64, 64, 64, F, F, nullptr, nullptr, nullptr, 0, nullptr), FP4Q_ERR_NULL);
    c = cfg();
    c.input_dtype = FP4Q_DTYPE_FP16;
    EXPECT(fp4_quantize(&c, F, 64, 64, 64, F, F, nullptr, nullptr, nullptr, 0, nullptr), FP4Q_ERR_DTYPE);
    c = cfg(FP4Q_NVFP4, FP4Q_TENSORWISE, 64);
    EXPECT(fp4_quantize(&c, F, 64, 64, 64, F, F, Ff, nullptr, nullptr, 0, nullptr), FP4Q_ERR_MODE);
    c = cfg(FP4Q_MXFP4, FP4Q_TENSORWISE);
    EXPECT(fp4_quantize(&c, F, 64, 64, 64, F, F, Ff, nullptr, nullptr, 0, nullptr), FP4Q_ERR_MODE);
    c = cfg(FP4Q_AMDFP4);
    c.scale_format = FP4Q_SCALE_E4M3;
    EXPECT(fp4_quantize(&c, F, 64, 64, 64, F, F, nullptr, nullptr, nullptr, 0, nullptr), FP4Q_ERR_MODE);
    c = cfg(FP4Q_NVFP4, FP4Q_OUTER_BLOCK, 24);
    EXPECT(fp4_quantize(&c, F, 64, 96, 96, F, F, Ff, nullptr, nullptr, 0, nullptr), FP4Q_ERR_SHAPE);
    c = cfg(FP4Q_NVFP4, FP4Q_OUTER_BLOCK, 128);
    EXPECT(fp4_quantize(&c, F, 64, 2880, 2880, F, F, Ff, nullptr, nullptr, 0, nullptr), FP4Q_ERR_SHAPE);
    c = cfg();
    EXPECT(fp4_quantize(&c, F, 64, 40, 40, F, F, nullptr, nullptr, nullptr, 0, nullptr), FP4Q_ERR_SHAPE);
    EXPECT(fp4_quantize(&c, F, 64, 64, 32, F, F, nullptr, nullptr, nullptr, 0, nullptr), FP4Q_ERR_SHAPE);
    EXPECT(fp4_quantize(&c, nullptr, 64, 64, 64, F, F, nullptr, nullptr, nullptr, 0, nullptr), FP4Q_ERR_NULL);
    EXPECT(fp4_quantize(&c, F, 64, 64, 64, F4, F, nullptr, nullptr, nullptr, 0, nullptr), FP4Q_ERR_ALIGN);
    EXPECT(fp4_quantize(&c, F, 0, 64, 64, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr), FP4Q_OK);
    c = cfg(FP4Q_NVFP4, FP4Q_TENSORWISE);
    const size_t ws = fp4q_workspace_bytes(&c, 64, 64);
    if (ws == 0) ++failures;
    EXPECT(fp4_quantize(&c, F, 64, 64, 64, F, F, Ff, nullptr, F, ws - 4, nullptr), FP4Q_ERR_WORKSPACE);
    EXPECT(fp4_qdq(&c, F, 64, 64, 64, nullptr, F, F, Ff, nullptr, F, ws, nullptr), FP4Q_ERR_NULL);
    c = cfg();
    EXPECT(fp4_qdq_noalloc(&c, F, 64, 64, 64, nullptr, F, F, nullptr, nullptr, nullptr), FP4Q_ERR_NULL);
    c = cfg(FP4Q_NVFP4, FP4Q_OUTER_BLOCK, 32, 1);
    EXPECT(fp4_quantize(&c, F, 64, 64, 64, F, F, Ff, nullptr, nullptr, 0, nullptr), FP4Q_ERR_UNSUPPORTED);

    // dequantise
    c = cfg(FP4Q_NVFP4, FP4Q_OUTER_BLOCK, 64);
    EXPECT(fp4_dequantize(&c, F, F, Ff, 64, 64, 1, F, nullptr), FP4Q_ERR_MODE);
    EXPECT(fp4_dequantize(&c, F, F, nullptr, 64, 64, 0, F, nullptr), FP4Q_ERR_NULL);
    EXPECT(fp4_dequantize(&c, F, F, Ff, 64, 48, 0, F, nullptr), FP4Q_ERR_SHAPE);

    // cast-transpose and grouped
    c = cfg();
    EXPECT(fp4_cast_transpose(&c, Fx, 40, 64, 64, F, F, nullptr, F, F, nullptr, nullptr, nullptr, 0, nullptr),
           FP4Q_ERR_SHAPE);
    c = cfg(FP4Q_MXFP4);
    EXPECT(fp4_cast_transpose(&c, Fx, 64, 64, 64, F, F, nullptr, F, F, nullptr, nullptr, nullptr, 0, nullptr),
           FP4Q_ERR_UNSUPPORTED);
    c = cfg(FP4Q_NVFP4, FP4Q_OUTER_BLOCK, 64);
    EXPECT(fp4_cast_transpose(&c, Fx, 64, 64, 64, F, F, Ff, F, F, nullptr, nullptr, nullptr, 0, nullptr),
           FP4Q_ERR_NULL);
    c = cfg(FP4Q_NVFP4, FP4Q_OUTER_BLOCK, 64, 1);
    EXPECT(fp4_cast_transpose(&c, Fx, 64, 64, 64, F, F, Ff, F, F, Ff + 1024, nullptr, nullptr, 0, nullptr),
           FP4Q_ERR_MODE);
    c = cfg(FP4Q_NVFP4, FP4Q_OUTER_BLOCK, 256);
    EXPECT(fp4_cast_transpose(&c, Fx, 256, 256, 256, F, F, Ff, F, F, Ff, nullptr, nullptr, 0, nullptr),
           FP4Q_ERR_UNSUPPORTED);
    std::vector<int64_t> rows = {64, 80};
    c = cfg(FP4Q_NVFP4, FP4Q_OUTER_BLOCK, 64, 1);
    EXPECT(fp4_cast_transpose_grouped(&c, 2, rows.data(), 64, Fx, 64, F, F, Ff, F, F, nullptr, nullptr, nullptr, 0,
                                      nullptr),
           FP4Q_ERR_SHAPE);
    EXPECT(fp4_cast_transpose_grouped(&c, 2, nullptr, 64, Fx, 64, F, F, Ff, F, F, nullptr, nullptr, nullptr, 0,
                                      nullptr),
           FP4Q_ERR_NULL);
    EXPECT(fp4_cast_transpose_grouped(&c, 0, nullptr, 64, Fx, 64, F, F, Ff, F, F, nullptr, nullptr, nullptr, 0,
                                      nullptr),
           FP4Q_OK);

    // size and workspace queries over many configurations and shapes
    const int formats[3] = {FP4Q_NVFP4, FP4Q_AMDFP4, FP4Q_MXFP4};
    const int tls[3] = {FP4Q_TWO_LEVEL_NONE, FP4Q_TENSORWISE, FP4Q_OUTER_BLOCK};
    const int obss[5] = {16, 32, 64, 128, 256};
    for (int f : formats)
        for (int tl : tls)
            for (int ob : obss)
                for (int o2d = 0; o2d < 2; ++o2d)
                    for (int64_t R : {0, 16, 64, 128, 2880, 16384})
                        for (int64_t Cc : {0, 32, 64, 256, 2880}) {
                            fp4q_cfg q = cfg(f, tl, tl == FP4Q_OUTER_BLOCK ? ob : 0, tl == FP4Q_OUTER_BLOCK ? o2d : 0);
                            fp4q_sizes sz;
                            (void)fp4q_buffer_sizes(&q, R, Cc, &sz);
                            (void)fp4q_workspace_bytes(&q, R, Cc);
                            std::vector<int64_t> g(70, R);
                            for (int w = 0; w < 2; ++w) {
                                (void)fp4q_cast_transpose_workspace_bytes(&q, 1, &R, Cc, w);
                                (void)fp4q_cast_transpose_workspace_bytes(&q, 70, g.data(), Cc, w);
                            }
                        }
    (void)fp4q_buffer_sizes(nullptr, 64, 64, nullptr);
    (void)fp4q_cast_transpose_workspace_bytes(nullptr, 1, nullptr, 64, 0);
    c = cfg();
    (void)fp4q_cast_transpose_workspace_bytes(&c, -1, nullptr, 64, 0);
    if (fp4q_mx_scales_tiled_bytes(0, 0) != 0) ++failures;

    // GEMM and MXFP4 projection rules
    c = cfg(FP4Q_MXFP4);
    EXPECT(fp4_mm(&c, F, F, F, F, 64, 64, 96, 0, F, 64, nullptr), FP4Q_ERR_SHAPE);
    EXPECT(fp4_mm(&c, F, F, F, F, 64, 64, 128, 3, F, 64, nullptr), FP4Q_ERR_MODE);
    EXPECT(fp4_mm(&c, F4, F, F, F, 64, 64, 128, 0, F, 64, nullptr), FP4Q_ERR_ALIGN);
    EXPECT(fp4_mx_scales_tiled(F, 64, 48, F, nullptr), FP4Q_ERR_SHAPE);
    EXPECT(fp4_mx_project_fp8(&c, Fx, 96, 128, 128, nullptr, nullptr, nullptr, nullptr, nullptr, F, nullptr, nullptr,
                              nullptr),
           FP4Q_ERR_SHAPE);
    c = cfg();
    EXPECT(fp4_mx_project_fp8(&c, Fx, 128, 128, 128, Fx, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                              nullptr),
           FP4Q_ERR_MODE);

    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("abi driver: every host path ran clean\n");
    return 0;
}
