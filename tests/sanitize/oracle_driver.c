/* oracle_driver.c -- runs every exported function of the C oracle
 * (oracle/fp4_oracle.c, test infrastructure) on small seeded inputs: every
 * NV / AMD mode (none, tensorwise, 1D and 2D outer, 16 x 16 inner tiles, RNE
 * and SR, error feedback, precomputed outer scales, binary32 sources and
 * targets, ragged and single-tile shapes), grouped calls with empty groups,
 * dequantisation of every outer kind, MXFP4 (bf16 and binary32, the FP8
 * re-encodings, the GEMM), and the format helpers.  Built with
 * -fsanitize=address,undefined by tests/test_sanitizers.py so that any
 * out-of-bounds access or undefined behaviour in the oracle aborts the run;
 * the results themselves are checked by the Python suite.  A few internal
 * consistency checks (grouped == single calls, dequantise == qdq output)
 * make sure the calls really ran. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t scale_fmt, two_level, obs, outer_2d, stochastic, use_given_outer, inner_2d;
    uint64_t seed, step, index_base;
} orc_nv_params;

float orc_bf16_to_f32(uint16_t b);
uint16_t orc_f32_to_bf16(float f);
double orc_e2m1_value(int m);
int orc_e2m1_rne(double a);
int orc_e2m1_sr(double a, uint32_t u16);
double orc_scale_decode(int sfmt, int c);
int orc_scale_encode(int sfmt, float y);
double orc_ue8m0_decode(int c);
void orc_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]);
uint32_t orc_sr_u16(uint64_t seed, uint64_t step, uint64_t idx);
void orc_sr_u16_array(uint64_t seed, uint64_t step, uint64_t idx0, int64_t n, uint16_t* out);
void orc_div_array(const float* a, const float* b, int64_t n, float* out);
int orc_nv_quantize_ex(const orc_nv_params* prm, const void* X, int x_f32, int64_t R, int64_t C, float* residual,
                       uint8_t* row_codes, uint8_t* row_scales, float* row_outer, void* row_y, uint8_t* col_codes,
                       uint8_t* col_scales, float* col_outer, void* col_y, int y_f32);
int orc_nv_quantize_grouped(const orc_nv_params* prm, int32_t G, const int64_t* rows, int64_t C, const uint16_t* X,
                            float* residual, uint8_t* row_codes, uint8_t* row_scales, float* row_outer,
                            uint8_t* col_codes, uint8_t* col_scales, float* col_outer);
int orc_nv_dequantize_ex(int sfmt, int outer_kind, int64_t obs, const uint8_t* codes, const uint8_t* scales,
                         const float* outer, int64_t R, int64_t C, void* y, int y_f32);
int orc_mx_qdq_ex(const void* X, int x_f32, int64_t R, int64_t C, uint8_t* codes, uint8_t* scales, void* y, int y_f32);
int orc_mx_dequantize_ex(const uint8_t* codes, const uint8_t* scales, int64_t R, int64_t C, void* y, int y_f32);
int orc_mx_project_encode(const uint16_t* X, int64_t R, int64_t C, uint16_t* y_out, uint8_t* mx8_row,
                          uint8_t* mx8_row_sc, uint8_t* mx8_col, uint8_t* mx8_col_sc, uint8_t* blk, uint8_t* blk_t,
                          float* blk_sc);
int orc_mx_mm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes, const uint8_t* b_scales,
              int64_t M, int64_t N, int64_t K, double* c, double* s);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void)
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (uint32_t)(rng_state >> 16);
}

/* bf16 patterns: mostly finite values of varied magnitude, some edge values */
static void fill_bf16(uint16_t* x, int64_t n)
{
    static const uint16_t edge[] = {0x0000, 0x8000, 0x0001, 0x8001, 0x0040, 0x7F7F, 0xFF7F, 0x7F80, 0xFF80, 0x7FC0};
    for (int64_t i = 0; i < n; ++i) {
        const uint32_t r = rnd();
        if (r % 61 == 0) x[i] = edge[(r >> 8) % 10];
        else x[i] = (uint16_t)((r & 0x8000u) | (0x3000u + ((r >> 4) % 0x1800u)));
    }
}

static void fill_f32(float* z, int64_t n, float scale)
{
    for (int64_t i = 0; i < n; ++i) z[i] = scale * ((float)(int32_t)(rnd() % 2001) - 1000.0f) / 1000.0f;
}

static int failures = 0;
#define CHECK(c)                                                            \
    do {                                                                    \
        if (!(c)) {                                                         \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                     \
        }                                                                   \
    } while (0)

static void nv_case(int sfmt, int two_level, int obs, int outer_2d, int sr, int ef, int inner_2d, int x_f32, int y_f32,
                    int64_t R, int64_t C)
{
    const int64_t N = R * C;
    void* X = malloc((size_t)N * (x_f32 ? 4 : 2));
    if (x_f32) fill_f32((float*)X, N, 3.0f);
    else fill_bf16((uint16_t*)X, N);
    float* res = ef ? (float*)malloc((size_t)N * 4) : NULL;
    if (res) fill_f32(res, N, 0.01f);
    const int64_t nro = two_level == 0 ? 0 : two_level == 1 ? 1 : outer_2d ? (R / obs) * (C / obs) : R * (C / obs);
    const int64_t nco = (two_level == 2 && !outer_2d) ? C * (R / obs) : 0;
    uint8_t* rc = malloc((size_t)(N / 2));
    uint8_t* rs = malloc((size_t)(N / 16));
    uint8_t* cc = malloc((size_t)(N / 2));
    uint8_t* cs = malloc((size_t)(N / 16));
    float* ro = nro ? malloc((size_t)nro * 4) : NULL;
    float* co = nco ? malloc((size_t)nco * 4) : NULL;
    void* ry = malloc((size_t)N * (y_f32 ? 4 : 2));
    void* cy = malloc((size_t)N * (y_f32 ? 4 : 2));
    orc_nv_params p = {sfmt, two_level, obs, outer_2d, sr, 0, inner_2d, 11, 3, 5};
    int rc0 = orc_nv_quantize_ex(&p, X, x_f32, R, C, res, rc, rs, ro, ry, cc, cs, co, cy, y_f32);
    CHECK(rc0 == 0);
    /* dequantise the rowwise buffers: must give the qdq output */
    void* y2 = malloc((size_t)N * (y_f32 ? 4 : 2));
    const int kind = two_level == 0 ? 0 : two_level == 1 ? 1 : outer_2d ? 3 : 2;
    CHECK(orc_nv_dequantize_ex(sfmt, kind, obs, rc, rs, ro, R, C, y2, y_f32) == 0);
    CHECK(memcmp(y2, ry, (size_t)N * (y_f32 ? 4 : 2)) == 0);
    /* precomputed outer scales reproduce the codes */
    if (two_level != 0 && !ef) {
        orc_nv_params q = p;
        q.use_given_outer = 1;
        uint8_t* rc2 = malloc((size_t)(N / 2));
        uint8_t* cc2 = malloc((size_t)(N / 2));
        CHECK(orc_nv_quantize_ex(&q, X, x_f32, R, C, NULL, rc2, rs, ro, NULL, cc2, cs, co, NULL, y_f32) == 0);
        CHECK(memcmp(rc2, rc, (size_t)(N / 2)) == 0);
        CHECK(memcmp(cc2, cc, (size_t)(N / 2)) == 0);
        free(rc2);
        free(cc2);
    }
    free(X); free(res); free(rc); free(rs); free(cc); free(cs); free(ro); free(co); free(ry); free(cy); free(y2);
}

int main(void)
{
    /* format helpers */
    for (int m = 0; m < 8; ++m) CHECK(orc_e2m1_rne(orc_e2m1_value(m)) == m);
    for (int c = 0; c < 256; ++c) {
        const double d1 = orc_scale_decode(1, c), d2 = orc_scale_decode(2, c);
        if (c < 0x7F) CHECK(orc_scale_encode(1, (float)d1) == c);
        if (c < 0xFF) CHECK(orc_scale_encode(2, (float)d2) == c);
        (void)orc_ue8m0_decode(c);
    }
    for (uint32_t u = 0; u < 65536; u += 97) (void)orc_e2m1_sr(2.3, u);
    for (int b = 0; b < 65536; b += 31) CHECK(orc_f32_to_bf16(orc_bf16_to_f32((uint16_t)b)) == (uint16_t)b ||
                                              ((b & 0x7FFF) > 0x7F80));
    uint32_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, out[4];
    orc_philox4x32_10(ctr, key, out);
    uint16_t u16[37];
    orc_sr_u16_array(7, 3, 5, 37, u16);
    for (int i = 0; i < 37; ++i) CHECK(u16[i] == orc_sr_u16(7, 3, 5 + (uint64_t)i));
    float a[33], bb[33], q[33];
    fill_f32(a, 33, 5.0f);
    fill_f32(bb, 33, 2.0f);
    for (int i = 0; i < 33; ++i) bb[i] = bb[i] == 0.0f ? 1.0f : bb[i];
    orc_div_array(a, bb, 33, q);

    /* NV / AMD modes: sfmt, two_level, obs, outer_2d, sr, ef, inner_2d, x_f32, y_f32, R, C */
    nv_case(1, 0, 0, 0, 0, 0, 0, 0, 0, 16, 16);
    nv_case(1, 0, 0, 0, 1, 1, 0, 0, 0, 48, 80);
    nv_case(1, 1, 0, 0, 0, 0, 0, 0, 0, 32, 48);
    nv_case(2, 1, 0, 0, 1, 1, 0, 1, 1, 32, 64);
    nv_case(1, 2, 16, 0, 0, 0, 0, 0, 0, 48, 80);
    nv_case(2, 2, 32, 0, 1, 1, 0, 0, 1, 64, 96);
    nv_case(1, 2, 64, 0, 1, 0, 0, 1, 0, 128, 192);
    nv_case(1, 2, 128, 0, 0, 1, 0, 0, 0, 128, 256);
    nv_case(1, 2, 16, 1, 0, 0, 0, 0, 0, 32, 48);
    nv_case(1, 2, 64, 1, 1, 1, 0, 0, 0, 128, 192);
    nv_case(2, 2, 64, 1, 0, 0, 1, 0, 0, 64, 128);
    nv_case(1, 0, 0, 0, 1, 1, 1, 0, 0, 48, 64);
    nv_case(1, 1, 0, 0, 0, 1, 1, 0, 0, 32, 32);

    /* grouped, with empty groups; must equal single calls */
    {
        const int64_t rows[5] = {64, 0, 128, 0, 64};
        const int64_t C = 128, R = 256, N = R * C;
        uint16_t* X = malloc((size_t)N * 2);
        fill_bf16(X, N);
        float* z1 = malloc((size_t)N * 4);
        float* z2 = malloc((size_t)N * 4);
        fill_f32(z1, N, 0.01f);
        memcpy(z2, z1, (size_t)N * 4);
        uint8_t *rc = malloc(N / 2), *rs = malloc(N / 16), *cc = malloc(N / 2), *cs = malloc(N / 16);
        float* ro = malloc((size_t)(N / 64 / 64) * 4);
        orc_nv_params p = {1, 2, 64, 1, 1, 0, 0, 5, 1, 0};
        CHECK(orc_nv_quantize_grouped(&p, 5, rows, C, X, z1, rc, rs, ro, cc, cs, NULL) == 0);
        /* group 2 alone */
        orc_nv_params p2 = p;
        p2.index_base = 64 * (uint64_t)C;
        uint8_t *rc2 = malloc(128 * C / 2), *rs2 = malloc(128 * C / 16), *cc2 = malloc(128 * C / 2),
                *cs2 = malloc(128 * C / 16);
        float* ro2 = malloc(4 * 4);
        CHECK(orc_nv_quantize_ex(&p2, X + 64 * C, 0, 128, C, z2 + 64 * C, rc2, rs2, ro2, NULL, cc2, cs2, NULL, NULL,
                                 0) == 0);
        CHECK(memcmp(rc2, rc + 64 * C / 2, 128 * C / 2) == 0);
        CHECK(memcmp(cc2, cc + 64 * C / 2, 128 * C / 2) == 0);
        CHECK(memcmp(z2 + 64 * C, z1 + 64 * C, 128 * C * 4) == 0);
        free(X); free(z1); free(z2); free(rc); free(rs); free(cc); free(cs); free(ro);
        free(rc2); free(rs2); free(cc2); free(cs2); free(ro2);
    }

    /* MXFP4: bf16 and binary32 sources, dequantise, FP8 re-encodings, GEMM */
    {
        const int64_t R = 128, C = 256, N = R * C;
        uint16_t* X = malloc((size_t)N * 2);
        fill_bf16(X, N);
        uint8_t *codes = malloc(N / 2), *scales = malloc(N / 32);
        uint16_t *y = malloc((size_t)N * 2), *y2 = malloc((size_t)N * 2);
        CHECK(orc_mx_qdq_ex(X, 0, R, C, codes, scales, y, 0) == 0);
        CHECK(orc_mx_dequantize_ex(codes, scales, R, C, y2, 0) == 0);
        CHECK(memcmp(y, y2, (size_t)N * 2) == 0);
        float* xf = malloc((size_t)N * 4);
        fill_f32(xf, N, 100.0f);
        float* yf = malloc((size_t)N * 4);
        CHECK(orc_mx_qdq_ex(xf, 1, R, C, codes, scales, yf, 1) == 0);
        uint8_t *r8 = malloc(N), *r8s = malloc(N / 32), *c8 = malloc(N), *c8s = malloc(N / 32), *b = malloc(N),
                *bt = malloc(N);
        float* bs = malloc((size_t)(N / 128 / 128) * 4);
        CHECK(orc_mx_project_encode(X, R, C, y2, r8, r8s, c8, c8s, b, bt, bs) == 0);
        CHECK(memcmp(y, y2, (size_t)N * 2) == 0);
        const int64_t M = 32, NN = 48, K = 256;
        uint8_t *ac = malloc(M * K / 2), *as = malloc(M * K / 32), *bc = malloc(NN * K / 2), *bsc = malloc(NN * K / 32);
        for (int64_t i = 0; i < M * K / 2; ++i) ac[i] = (uint8_t)rnd();
        for (int64_t i = 0; i < NN * K / 2; ++i) bc[i] = (uint8_t)rnd();
        for (int64_t i = 0; i < M * K / 32; ++i) as[i] = (uint8_t)(120 + rnd() % 16);
        for (int64_t i = 0; i < NN * K / 32; ++i) bsc[i] = (uint8_t)(120 + rnd() % 16);
        double* c = malloc((size_t)(M * NN) * 8);
        double* sm = malloc((size_t)(M * NN) * 8);
        CHECK(orc_mx_mm(ac, as, bc, bsc, M, NN, K, c, sm) == 0);
        free(X); free(codes); free(scales); free(y); free(y2); free(xf); free(yf);
        free(r8); free(r8s); free(c8); free(c8s); free(b); free(bt); free(bs);
        free(ac); free(as); free(bc); free(bsc); free(c); free(sm);
    }
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle driver: every entry point ran clean\n");
    return 0;
}
