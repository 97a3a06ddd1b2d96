/* Drives every entry point of oracle/oracle.c on small inputs, single- and multi-threaded, with
 * self-checks, for the sanitizer builds (AddressSanitizer + UndefinedBehaviorSanitizer, and
 * ThreadSanitizer on the thread pool). Exit status 0 when every check holds. Test infrastructure. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_unpack_codes(const uint32_t*, int64_t, int64_t, int, uint8_t*);
int orc_pack_codes(const uint8_t*, int64_t, int64_t, int, uint32_t*);
void orc_bf16_to_f32(const uint16_t*, int64_t, float*);
void orc_f32_to_bf16(const float*, int64_t, uint16_t*);
void orc_f16_to_f32(const uint16_t*, int64_t, float*);
void orc_f32_to_f16(const float*, int64_t, uint16_t*);
int orc_dequantize(const uint32_t*, const uint16_t*, const uint16_t*, int64_t, int64_t, int64_t, int, float*, int);
int orc_dequant_rows(const uint32_t*, const uint16_t*, const uint16_t*, int64_t, int64_t, int64_t, int,
                     const uint32_t*, int64_t, float*, int);
int orc_qmm(const void*, int, int64_t, const uint32_t*, const uint16_t*, const uint16_t*, int64_t, int64_t, int64_t,
            int, double*, int);
void orc_silu_gate(const uint16_t*, const uint16_t*, int64_t, double*);
int orc_silu_gate_qmm(const uint16_t*, const uint16_t*, const uint16_t*, int64_t, const uint32_t*, const uint16_t*,
                      const uint16_t*, int64_t, int64_t, int64_t, int, double*, int);
int orc_gather_qmm(const void*, int, int64_t, int64_t, const uint32_t*, const uint16_t*, const uint16_t*, int64_t,
                   int64_t, int64_t, int64_t, int, const uint32_t*, const uint32_t*, int64_t, double*, int);
int orc_quantize(const void*, int, int64_t, int64_t, int64_t, int, uint32_t*, uint16_t*, uint16_t*);
int orc_qmm_nt(const void*, int, int64_t, const uint32_t*, const uint16_t*, const uint16_t*, int64_t, int64_t,
               int64_t, int, double*);
int orc_dequantize_typed(const uint32_t*, const void*, const void*, int, int64_t, int64_t, int64_t, int, float*);
int orc_qmm_typed(const void*, int, int64_t, const uint32_t*, const void*, const void*, int, int64_t, int64_t,
                  int64_t, int, double*);

static int failures = 0;
#define CHECK(c)                                                              \
    do {                                                                      \
        if (!(c)) {                                                           \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);  \
            ++failures;                                                       \
        }                                                                     \
    } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) { /* xorshift64* */
    rng_state ^= rng_state >> 12; rng_state ^= rng_state << 25; rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static uint16_t bf16_of(float f) { uint32_t u; memcpy(&u, &f, 4); return (uint16_t)(u >> 16); }

int main(void) {
    const int widths[] = {1, 2, 3, 4, 5, 6, 8};
    const int64_t rows = 7, cols = 256, m = 3;
    for (int wi = 0; wi < 7; ++wi) {
        const int bits = widths[wi];
        for (int64_t group = 32; group <= 128; group *= 2) {
            const int64_t words = cols * bits / 32, groups = cols / group;
            uint8_t* codes = malloc((size_t)(rows * cols));
            uint8_t* back = malloc((size_t)(rows * cols));
            uint32_t* packed = malloc(sizeof(uint32_t) * (size_t)(rows * words));
            uint16_t* sc = malloc(2 * (size_t)(rows * groups));
            uint16_t* bi = malloc(2 * (size_t)(rows * groups));
            float* w = malloc(sizeof(float) * (size_t)(rows * cols));
            float* w2 = malloc(sizeof(float) * (size_t)(rows * cols));
            for (int64_t i = 0; i < rows * cols; ++i) codes[i] = (uint8_t)(rnd() & ((1u << bits) - 1));
            for (int64_t i = 0; i < rows * groups; ++i) {
                sc[i] = bf16_of(1e-3f + (float)(rnd() % 1000) * 2e-5f);
                bi[i] = bf16_of(-0.15f * (float)(rnd() % 1000) / 1000.f);
            }
            CHECK(orc_pack_codes(codes, rows, cols, bits, packed) == 0);
            CHECK(orc_unpack_codes(packed, rows, cols, bits, back) == 0);
            CHECK(memcmp(codes, back, (size_t)(rows * cols)) == 0);
            CHECK(orc_dequantize(packed, sc, bi, rows, cols, group, bits, w, 1) == 0);
            CHECK(orc_dequantize(packed, sc, bi, rows, cols, group, bits, w2, 4) == 0);
            CHECK(memcmp(w, w2, sizeof(float) * (size_t)(rows * cols)) == 0);
            /* gathered rows, an out-of-range index among them */
            const uint32_t idx[5] = {6, 0, 3, 3, 99};
            float* g = malloc(sizeof(float) * (size_t)(5 * cols));
            CHECK(orc_dequant_rows(packed, sc, bi, rows, cols, group, bits, idx, 5, g, 3) == 0);
            CHECK(memcmp(g, w + 6 * cols, sizeof(float) * (size_t)cols) == 0);
            CHECK(isnan(g[4 * cols]));
            /* qmm: float32 and bf16 x, threads 1 and 4 agree */
            float* xf = malloc(sizeof(float) * (size_t)(m * cols));
            uint16_t* xb = malloc(2 * (size_t)(m * cols));
            for (int64_t i = 0; i < m * cols; ++i) {
                xf[i] = (float)((int)(rnd() % 2001) - 1000) / 500.f;
                xb[i] = bf16_of(xf[i]);
            }
            double* y1 = malloc(sizeof(double) * (size_t)(m * rows));
            double* y4 = malloc(sizeof(double) * (size_t)(m * rows));
            CHECK(orc_qmm(xf, 0, m, packed, sc, bi, rows, cols, group, bits, y1, 1) == 0);
            CHECK(orc_qmm(xf, 0, m, packed, sc, bi, rows, cols, group, bits, y4, 4) == 0);
            CHECK(memcmp(y1, y4, sizeof(double) * (size_t)(m * rows)) == 0);
            CHECK(orc_qmm(xb, 1, m, packed, sc, bi, rows, cols, group, bits, y4, 2) == 0);
            /* fused product with and without a residual */
            uint16_t* resid = malloc(2 * (size_t)(m * rows));
            for (int64_t i = 0; i < m * rows; ++i) resid[i] = bf16_of(0.5f);
            CHECK(orc_silu_gate_qmm(xb, xb, resid, m, packed, sc, bi, rows, cols, group, bits, y1, 3) == 0);
            CHECK(orc_silu_gate_qmm(xb, xb, NULL, m, packed, sc, bi, rows, cols, group, bits, y4, 3) == 0);
            /* gathered products: two x batches of m rows against the weight taken as one batch */
            double* yg = malloc(sizeof(double) * (size_t)(3 * m * rows));
            const uint32_t lhs[3] = {1, 0, 5}, rhs[3] = {0, 0, 0};
            float* x2 = malloc(sizeof(float) * (size_t)(2 * m * cols));
            memcpy(x2, xf, sizeof(float) * (size_t)(m * cols));
            memcpy(x2 + m * cols, xf, sizeof(float) * (size_t)(m * cols));
            CHECK(orc_gather_qmm(x2, 0, 2, m, packed, sc, bi, 1, rows, cols, group, bits, lhs, rhs, 3, yg, 2) == 0);
            CHECK(isnan(yg[2 * m * rows]));
            /* without the transpose: the weight read as [rows (k), cols (n)] */
            double* ynt = malloc(sizeof(double) * (size_t)(2 * cols));
            float* xk = malloc(sizeof(float) * (size_t)(2 * rows));
            for (int64_t i = 0; i < 2 * rows; ++i) xk[i] = (float)i - 3.f;
            CHECK(orc_qmm_nt(xk, 0, 2, packed, sc, bi, rows, cols, group, bits, ynt) == 0);
            /* other float types */
            uint16_t* s16 = malloc(2 * (size_t)(rows * groups));
            uint16_t* b16 = malloc(2 * (size_t)(rows * groups));
            float* sf = malloc(sizeof(float) * (size_t)(rows * groups));
            float* bf = malloc(sizeof(float) * (size_t)(rows * groups));
            orc_bf16_to_f32(sc, rows * groups, sf);
            orc_bf16_to_f32(bi, rows * groups, bf);
            orc_f32_to_f16(sf, rows * groups, s16);
            orc_f32_to_f16(bf, rows * groups, b16);
            CHECK(orc_dequantize_typed(packed, sc, bi, 1, rows, cols, group, bits, w2) == 0);
            CHECK(memcmp(w, w2, sizeof(float) * (size_t)(rows * cols)) == 0);
            CHECK(orc_dequantize_typed(packed, s16, b16, 2, rows, cols, group, bits, w2) == 0);
            CHECK(orc_dequantize_typed(packed, sf, bf, 0, rows, cols, group, bits, w2) == 0);
            CHECK(orc_qmm_typed(xb, 1, m, packed, s16, b16, 2, rows, cols, group, bits, y1) == 0);
            /* quantize the dequantized weight back (float32 and bf16 input) */
            uint32_t* qp = malloc(sizeof(uint32_t) * (size_t)(rows * words));
            uint16_t* qs = malloc(2 * (size_t)(rows * groups));
            uint16_t* qb = malloc(2 * (size_t)(rows * groups));
            CHECK(orc_quantize(w, 0, rows, cols, group, bits, qp, qs, qb) == 0);
            uint16_t* wb16 = malloc(2 * (size_t)(rows * cols));
            orc_f32_to_bf16(w, rows * cols, wb16);
            CHECK(orc_quantize(wb16, 1, rows, cols, group, bits, qp, qs, qb) == 0);
            free(codes); free(back); free(packed); free(sc); free(bi); free(w); free(w2); free(g);
            free(xf); free(xb); free(y1); free(y4); free(resid); free(yg); free(x2); free(ynt); free(xk);
            free(s16); free(b16); free(sf); free(bf); free(qp); free(qs); free(qb); free(wb16);
        }
    }
    /* special values through the conversions and quantize: NaN, infinities, zeros, subnormals */
    float sp[64];
    for (int i = 0; i < 64; ++i) sp[i] = (float)i;
    sp[1] = NAN; sp[2] = INFINITY; sp[3] = -INFINITY; sp[4] = -0.0f; sp[5] = 1e-40f; sp[6] = 3e38f;
    uint16_t h[64];
    float back[64];
    orc_f32_to_bf16(sp, 64, h);
    orc_bf16_to_f32(h, 64, back);
    orc_f32_to_f16(sp, 64, h);
    orc_f16_to_f32(h, 64, back);
    uint32_t qp[8];
    uint16_t qs[2], qb[2];
    CHECK(orc_quantize(sp, 0, 1, 64, 32, 4, qp, qs, qb) == 0);
    /* parameters outside the format are refused */
    CHECK(orc_dequantize(qp, qs, qb, 1, 48, 32, 4, back, 1) == -1);
    CHECK(orc_quantize(sp, 0, 1, 64, 32, 9, qp, qs, qb) == -1);
    /* empty shapes */
    CHECK(orc_qmm(sp, 0, 0, qp, qs, qb, 0, 64, 32, 4, NULL, 4) == 0);
    CHECK(orc_dequant_rows(qp, qs, qb, 1, 64, 32, 4, NULL, 0, NULL, 4) == 0);
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle driver: all checks passed\n");
    return 0;
}
