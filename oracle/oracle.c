/*
 * CPU oracle for MLX-style grouped affine quantization:
 *   - dequantize:        w[n,k] = scale[n,k/G] * code[n,k] + bias[n,k/G]
 *   - gathered rows:     out[i,:] = dequantize(table)[idx[i], :]
 *   - quantized matmul:  y[m,n] = sum_k x[m,k] * w[n,k]      (y = x . dequantize(W)^T)
 *   - without transpose: y[m,n] = sum_k x[m,k] * w[k,n]      (y = x . dequantize(W), W [k, n])
 *   - gathered matmul:   y[i] = x[lhs[i]] . dequantize(W[rhs[i]])^T  (mixture-of-experts batches)
 *   - quantize:          bias = group min, scale = (max - min) / (2^bits - 1), code =
 *                        round((w - bias) / scale) clamped to [0, 2^bits - 1]
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline leg
 * may load this library. The HIP library never calls it and shares no code, header, table or
 * helper with it.
 *
 * It is plain and slow on purpose, so that it can be checked against the pages by eye:
 *   - a code is read one bit at a time out of the row's bit stream;
 *   - a weight is formed by the affine rule exactly as written: float32 product, then float32 sum;
 *   - matmul sums run sequentially over k in double precision, with no blocking or reordering.
 * Build with gcc -O2 -ffp-contract=off (no -ffast-math), so the compiler fuses nothing.
 *
 * Sources (the pages this follows):
 *   [moshi]  rlx-moshi, src/mlx_dequant.rs: doc comment and body of `dequantize_affine`
 *            (codes packed LSB-first, code s in bits [s*bits, (s+1)*bits); w = scale*code + bias
 *            with bias the group minimum; rows independent), and `bf16_to_f32` (widening by a
 *            16-bit left shift).
 *   [nuvec]  nuvec_core, quantized.rs: module documentation (codes form one little-endian bit
 *            stream per row stored as uint32; scales and biases are [.., in/group]), `check_params`
 *            (group sizes, bit widths), `dequantize` and `quantized_matmul` (x . dequantize(w)^T
 *            without materialising the dequantized matrix), `gather_indices` (indices as uint32;
 *            either index array defaults to every batch in order) and `gather_qmm` (output batch i
 *            is x[lhs[i]] . dequantize(w[rhs[i]])^T over flattened batch dimensions), module
 *            documentation of quantization (a value is stored as round((w - bias) / scale),
 *            clamped to [0, 2^bits - 1]) and `quantize`.
 *   [maya2]  maya2_mlx, quant.py: `mm` (x @ W.T for a quantized weight) and `rows` (an embedding
 *            lookup that dequantizes only the gathered rows).
 *   [spark]  spark_runtime, weights/mlx_int8.rs: module documentation (8-bit words hold four bytes,
 *            low byte = column 0; the affine formula per group of G columns); the fused decode
 *            products `gemv_gate_up` (two projections of one x), `gemv_silu_gate`
 *            (y = W . (silu(gate) * up)) and `gemv_silu_gate_resid` (the same plus a residual).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_VERSION 1

int orc_version(void) { return ORACLE_VERSION; }

/* ---- bf16 <-> f32 ----------------------------------------------------------------------- */

/* [moshi] bf16_to_f32: the bf16 bit pattern is the upper half of the float32 one. Exact. */
static float bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* float32 -> bf16, round to nearest, ties to even. The pages round no output themselves (the
 * moshi helper only truncates exactly representable test values); IEEE RNE is the plain reading
 * for bf16 outputs. The dropped low half decides: above the midpoint rounds up, below rounds
 * down, exactly the midpoint rounds to the even neighbour. A carry out of the mantissa steps the
 * exponent, which is again correct (and turns the largest finite values into infinity). NaN stays
 * NaN: its quiet bit is set so that dropping the payload's low half cannot turn it into infinity. */
static uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t hi = u >> 16;
    uint32_t lo = u & 0xffffu;
    if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u)))
        hi += 1;
    return (uint16_t)hi;
}

void orc_bf16_to_f32(const uint16_t* in, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_to_f32(in[i]);
}

void orc_f32_to_bf16(const float* in, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(in[i]);
}

/* ---- codes ------------------------------------------------------------------------------ */

/* [nuvec] module doc, [moshi] doc comment: a row is one little-endian bit stream; code j
 * occupies stream bits [j*bits, (j+1)*bits), least significant bit first. Stream bit p is bit
 * (p mod 32) of word (p div 32). Read one bit at a time, so a code that straddles two words
 * needs no special case. */
static uint32_t code_at(const uint32_t* row, int64_t j, int bits) {
    uint32_t code = 0;
    for (int t = 0; t < bits; ++t) {
        int64_t p = j * bits + t;
        uint32_t bit = (row[p / 32] >> (p % 32)) & 1u;
        code |= bit << t;
    }
    return code;
}

static int valid_stream(int64_t cols, int bits) {
    return bits >= 1 && bits <= 8 && cols >= 0 && (cols * bits) % 32 == 0;
}

/* codes [rows, cols] (one byte each) from packed [rows, cols*bits/32]. */
int orc_unpack_codes(const uint32_t* packed, int64_t rows, int64_t cols, int bits, uint8_t* codes) {
    if (!valid_stream(cols, bits)) return -1;
    int64_t words = cols * bits / 32;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < cols; ++j)
            codes[r * cols + j] = (uint8_t)code_at(packed + r * words, j, bits);
    return 0;
}

/* The exact inverse of orc_unpack_codes: writes every stream bit of each code, one by one.
 * Bits of a code above `bits` are ignored. */
int orc_pack_codes(const uint8_t* codes, int64_t rows, int64_t cols, int bits, uint32_t* packed) {
    if (!valid_stream(cols, bits)) return -1;
    int64_t words = cols * bits / 32;
    memset(packed, 0, (size_t)(rows * words) * sizeof(uint32_t));
    for (int64_t r = 0; r < rows; ++r) {
        uint32_t* row = packed + r * words;
        for (int64_t j = 0; j < cols; ++j)
            for (int t = 0; t < bits; ++t) {
                int64_t p = j * bits + t;
                if ((codes[r * cols + j] >> t) & 1u) row[p / 32] |= 1u << (p % 32);
            }
    }
    return 0;
}

/* ---- dequantize ------------------------------------------------------------------------- */

/* [moshi] body of dequantize_affine, [spark] module formula: w = scale * code + bias, where scale
 * and bias belong to the code's group g = col / G of its row. The product is formed in float32
 * and then the bias is added in float32 (two roundings as written; with bf16 scales and codes of
 * at most 8 bits the product is exact, so only the sum rounds). */
static float dequant_one(const uint32_t* prow, const uint16_t* srow, const uint16_t* brow,
                         int64_t col, int64_t group, int bits) {
    uint32_t code = code_at(prow, col, bits);
    int64_t g = col / group;
    float s = bf16_to_f32(srow[g]);
    float b = bf16_to_f32(brow[g]);
    float p = s * (float)code;
    float w = p + b;
    return w;
}

static void dequant_row(const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                        int64_t r, int64_t cols, int64_t group, int bits, float* out_row) {
    int64_t words = cols * bits / 32, groups = cols / group;
    const uint32_t* prow = packed + r * words;
    const uint16_t* srow = scales + r * groups;
    const uint16_t* brow = biases + r * groups;
    for (int64_t c = 0; c < cols; ++c)
        out_row[c] = dequant_one(prow, srow, brow, c, group, bits);
}

static int valid_params(int64_t cols, int64_t group, int bits) {
    /* [moshi] argument checks: group > 0 divides cols. Any bit width 1..8 is accepted here (the
     * oracle is wider than the library on purpose, so the pages' G = 8 example runs as given). */
    return valid_stream(cols, bits) && group > 0 && cols % group == 0;
}

/* ---- a tiny row-range thread pool ------------------------------------------------------- */

typedef void (*range_fn)(void* ctx, int64_t begin, int64_t end);
typedef struct { range_fn fn; void* ctx; int64_t begin, end; } range_job;

static void* range_entry(void* p) {
    range_job* j = (range_job*)p;
    j->fn(j->ctx, j->begin, j->end);
    return NULL;
}

/* Splits [0, total) into `threads` contiguous ranges and runs fn on each. */
static void run_ranges(range_fn fn, void* ctx, int64_t total, int threads) {
    if (threads < 1) threads = 1;
    if (threads > total) threads = (int)(total > 0 ? total : 1);
    if (threads == 1) { fn(ctx, 0, total); return; }
    pthread_t* tid = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)threads);
    range_job* jobs = (range_job*)malloc(sizeof(range_job) * (size_t)threads);
    for (int t = 0; t < threads; ++t) {
        jobs[t].fn = fn;
        jobs[t].ctx = ctx;
        jobs[t].begin = total * t / threads;
        jobs[t].end = total * (t + 1) / threads;
        pthread_create(&tid[t], NULL, range_entry, &jobs[t]);
    }
    for (int t = 0; t < threads; ++t) pthread_join(tid[t], NULL);
    free(tid);
    free(jobs);
}

typedef struct {
    const uint32_t* packed; const uint16_t* scales; const uint16_t* biases;
    int64_t cols, group; int bits;
    const uint32_t* idx; int64_t table_rows;
    float* out;
} dq_ctx;

static void dq_range(void* p, int64_t b, int64_t e) {
    dq_ctx* c = (dq_ctx*)p;
    for (int64_t r = b; r < e; ++r)
        dequant_row(c->packed, c->scales, c->biases, r, c->cols, c->group, c->bits, c->out + r * c->cols);
}

/* out float32 [rows, cols]. Returns 0, or -1 for parameters outside the format. */
int orc_dequantize(const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                   int64_t rows, int64_t cols, int64_t group, int bits, float* out, int threads) {
    if (rows < 0 || !valid_params(cols, group, bits)) return -1;
    dq_ctx c = {packed, scales, biases, cols, group, bits, NULL, 0, out};
    run_ranges(dq_range, &c, rows, threads);
    return 0;
}

/* [maya2] rows: dequantize only the gathered rows; [nuvec] gather_indices: indices are uint32.
 * An index past the table (the pages do not say) gives a row of quiet NaNs. */
static void rows_range(void* p, int64_t b, int64_t e) {
    dq_ctx* c = (dq_ctx*)p;
    uint32_t qnan_bits = 0x7fc00000u;
    float qnan;
    memcpy(&qnan, &qnan_bits, sizeof qnan);
    for (int64_t i = b; i < e; ++i) {
        float* o = c->out + i * c->cols;
        int64_t r = (int64_t)c->idx[i];
        if (r >= c->table_rows) {
            for (int64_t j = 0; j < c->cols; ++j) o[j] = qnan;
        } else {
            dequant_row(c->packed, c->scales, c->biases, r, c->cols, c->group, c->bits, o);
        }
    }
}

int orc_dequant_rows(const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                     int64_t table_rows, int64_t cols, int64_t group, int bits,
                     const uint32_t* idx, int64_t n_idx, float* out, int threads) {
    if (table_rows < 0 || n_idx < 0 || !valid_params(cols, group, bits)) return -1;
    dq_ctx c = {packed, scales, biases, cols, group, bits, idx, table_rows, out};
    run_ranges(rows_range, &c, n_idx, threads);
    return 0;
}

/* ---- quantized matmul ------------------------------------------------------------------- */

/* [nuvec] quantized_matmul with transpose (weights stored [out, in]), [maya2] mm:
 *   y[m, n] = sum over k of x[m, k] * w[n, k],  w = the dequantized weight above.
 * x is float32, or bf16 widened exactly. Each product and the running sum are in double and the
 * sum runs over k in order. The result is returned in double; rounding it to the caller's output
 * type is the comparison's business. */
typedef struct {
    const double* xd; int64_t m;
    const uint32_t* packed; const uint16_t* scales; const uint16_t* biases;
    int64_t n, k, group; int bits;
    double* out;
} qmm_ctx;

static void qmm_range(void* p, int64_t b, int64_t e) {
    qmm_ctx* c = (qmm_ctx*)p;
    float* w = (float*)malloc(sizeof(float) * (size_t)(c->k > 0 ? c->k : 1));
    for (int64_t nn = b; nn < e; ++nn) {
        dequant_row(c->packed, c->scales, c->biases, nn, c->k, c->group, c->bits, w);
        for (int64_t mm = 0; mm < c->m; ++mm) {
            const double* xr = c->xd + mm * c->k;
            double acc = 0.0;
            for (int64_t kk = 0; kk < c->k; ++kk) acc += xr[kk] * (double)w[kk];
            c->out[mm * c->n + nn] = acc;
        }
    }
    free(w);
}

/* x [m, k] (float32, or bf16 bits when x_is_bf16), packed [n, k*bits/32], scales/biases
 * [n, k/group] bf16 bits; out double [m, n]. Returns 0, or -1 for parameters outside the format. */
int orc_qmm(const void* x, int x_is_bf16, int64_t m, const uint32_t* packed, const uint16_t* scales,
            const uint16_t* biases, int64_t n, int64_t k, int64_t group, int bits, double* out,
            int threads) {
    if (m < 0 || n < 0 || !valid_params(k, group, bits)) return -1;
    double* xd = (double*)malloc(sizeof(double) * (size_t)(m * k > 0 ? m * k : 1));
    if (!xd) return -2;
    for (int64_t i = 0; i < m * k; ++i)
        xd[i] = x_is_bf16 ? (double)bf16_to_f32(((const uint16_t*)x)[i]) : (double)((const float*)x)[i];
    qmm_ctx c = {xd, m, packed, scales, biases, n, k, group, bits, out};
    run_ranges(qmm_range, &c, n, threads);
    free(xd);
    return 0;
}

/* ---- fused decode products --------------------------------------------------------------- */

/* silu(v) = v * sigmoid(v) = v / (1 + exp(-v)), in double. */
static double silu(double v) { return v / (1.0 + exp(-v)); }

/* [spark] the activation of gemv_silu_gate: h = silu(gate) * up, element by element, with gate and
 * up bf16 bit patterns widened exactly; h in double. */
void orc_silu_gate(const uint16_t* gate, const uint16_t* up, int64_t count, double* out) {
    for (int64_t i = 0; i < count; ++i)
        out[i] = silu((double)bf16_to_f32(gate[i])) * (double)bf16_to_f32(up[i]);
}

/* [spark] gemv_silu_gate (resid null) and gemv_silu_gate_resid:
 *   y[m, n] = sum over k of h[m, k] * w[n, k]  (+ resid[m, n]),  h = silu(gate) * up,
 * gate and up [m, k] and resid [m, n] bf16 bit patterns; everything after the widening in double,
 * the sum over k in order. Returns 0, or -1 for parameters outside the format. */
int orc_silu_gate_qmm(const uint16_t* gate, const uint16_t* up, const uint16_t* resid, int64_t m,
                      const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                      int64_t n, int64_t k, int64_t group, int bits, double* out, int threads) {
    if (m < 0 || n < 0 || !valid_params(k, group, bits)) return -1;
    double* h = (double*)malloc(sizeof(double) * (size_t)(m * k > 0 ? m * k : 1));
    if (!h) return -2;
    orc_silu_gate(gate, up, m * k, h);
    qmm_ctx c = {h, m, packed, scales, biases, n, k, group, bits, out};
    run_ranges(qmm_range, &c, n, threads);
    if (resid)
        for (int64_t i = 0; i < m * n; ++i) out[i] += (double)bf16_to_f32(resid[i]);
    free(h);
    return 0;
}

/* [nuvec] gather_qmm (transpose form): x is [x_batches, m, k] (bf16 bit patterns or float32), the
 * weight is w_batches matrices of [n, k] with their scales and biases stacked the same way, and
 * output batch i (of `batch`) is
 *     y[i] = x[lhs[i]] . dequantize(W[rhs[i]])^T          ([m, n], double)
 * computed by orc_qmm on that pair. [nuvec] gather_indices: a null index array stands for
 * 0, 1, ..., batch - 1. The pages leave an index past its operand undefined; here that output
 * batch is NaN. `sorted_indices` only promises an order of rhs that lets a kernel walk each weight
 * batch once: it changes no value, so the oracle has no such argument.
 * Returns 0, or -1 for parameters outside the format. */
int orc_gather_qmm(const void* x, int x_is_bf16, int64_t x_batches, int64_t m, const uint32_t* packed,
                   const uint16_t* scales, const uint16_t* biases, int64_t w_batches, int64_t n, int64_t k,
                   int64_t group, int bits, const uint32_t* lhs, const uint32_t* rhs, int64_t batch,
                   double* out, int threads) {
    if (m < 0 || n < 0 || batch < 0 || x_batches < 0 || w_batches < 0 || !valid_params(k, group, bits))
        return -1;
    if ((!lhs && batch > x_batches) || (!rhs && batch > w_batches)) return -1;
    const int64_t xsize = x_is_bf16 ? 2 : 4;
    const int64_t words = k * bits / 32; /* packed words per weight row */
    for (int64_t i = 0; i < batch; ++i) {
        const int64_t li = lhs ? (int64_t)lhs[i] : i;
        const int64_t ri = rhs ? (int64_t)rhs[i] : i;
        double* yi = out + i * m * n;
        if (li >= x_batches || ri >= w_batches) {
            for (int64_t t = 0; t < m * n; ++t) yi[t] = NAN;
            continue;
        }
        const void* xi = (const uint8_t*)x + li * m * k * xsize;
        int rc = orc_qmm(xi, x_is_bf16, m, packed + ri * n * words, scales + ri * n * (k / group),
                         biases + ri * n * (k / group), n, k, group, bits, yi, threads);
        if (rc != 0) return rc;
    }
    return 0;
}

/* Sign (-1, 0, +1) of the exact sum a + b + c of three doubles, by expansion arithmetic
 * (Shewchuk, "Adaptive precision floating-point arithmetic and fast robust geometric predicates",
 * 1997: Two-Sum, and Grow-Expansion with its theorem that the result is a nonoverlapping expansion
 * in increasing order of magnitude, so its sign is that of its largest nonzero component).
 * Round-to-nearest double arithmetic, no overflow (the arguments are float32-sized). */
static void two_sum(double a, double b, double* s, double* e) {
    *s = a + b;
    const double bv = *s - a;
    const double av = *s - bv;
    *e = (a - av) + (b - bv);
}

static int sign_of_sum3(double a, double b, double c) {
    double x, ex, q, h1, h2;
    two_sum(a, b, &x, &ex);  /* a + b = x + ex exactly: the expansion [ex, x] */
    two_sum(c, ex, &q, &h1); /* grow it by c */
    two_sum(q, x, &q, &h2);  /* a + b + c = h1 + h2 + q exactly */
    if (q != 0.0) return q > 0.0 ? 1 : -1; /* a NaN lands here as -1 */
    if (h2 != 0.0) return h2 > 0.0 ? 1 : -1;
    return (h1 > 0.0) - (h1 < 0.0);
}

/* [nuvec] quantized_matmul without the transpose: y = x . dequantize(w), for a weight stored
 * [k, n] (its rows are the k index, each a bit stream of n codes in groups of G along n):
 *     y[m, n] = sum over k of x[m, k] * w[k, n]
 * in double, sequentially in k, with each row of w dequantized as everywhere else. x [m, k]
 * (float32 or bf16 bits), packed [k, n*bits/32], scales/biases [k, n/group]; out double [m, n].
 * Returns 0, or -1 for parameters outside the format. */
int orc_qmm_nt(const void* x, int x_is_bf16, int64_t m, const uint32_t* packed, const uint16_t* scales,
               const uint16_t* biases, int64_t k, int64_t n, int64_t group, int bits, double* out) {
    if (m < 0 || k < 0 || !valid_params(n, group, bits)) return -1;
    float* w = (float*)malloc(sizeof(float) * (size_t)(k * n > 0 ? k * n : 1));
    if (!w) return -2;
    for (int64_t kk = 0; kk < k; ++kk) dequant_row(packed, scales, biases, kk, n, group, bits, w + kk * n);
    for (int64_t mm = 0; mm < m; ++mm)
        for (int64_t nn = 0; nn < n; ++nn) {
            double acc = 0.0;
            for (int64_t kk = 0; kk < k; ++kk) {
                const int64_t i = mm * k + kk;
                const double xv = x_is_bf16 ? (double)bf16_to_f32(((const uint16_t*)x)[i]) : (double)((const float*)x)[i];
                acc += xv * (double)w[kk * n + nn];
            }
            out[mm * n + nn] = acc;
        }
    free(w);
    return 0;
}

/* ---- other float types of x, scales and biases -------------------------------------------- */

/* [nuvec] quantized_matmul and dequantize promote x, scales and biases to one float type, and
 * scales keep the weight's dtype (float16, bfloat16 or float32). dtype codes: 0 float32,
 * 1 bfloat16 (bits), 2 float16 (bits). */

/* IEEE binary16 -> float32, exact: sign, 5-bit exponent (bias 15), 10-bit fraction; exponent 0 is
 * zero or subnormal (fraction * 2^-24), exponent 31 is infinity or NaN. */
static float f16_to_f32(uint16_t h) {
    const int sign = (h >> 15) & 1;
    const int e = (h >> 10) & 31;
    const int f = h & 1023;
    float v;
    if (e == 0) v = ldexpf((float)f, -24);
    else if (e == 31) v = f ? NAN : INFINITY;
    else v = ldexpf((float)(1024 + f), e - 25);
    return sign ? -v : v;
}

void orc_f16_to_f32(const uint16_t* in, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = f16_to_f32(in[i]);
}

/* float32 -> binary16, round to nearest, ties to even: the value is scaled to an integer count of
 * the target's units (2^-24 below 2^-14, else 2^(e-10) for its binade), rounded with ties to
 * even, and re-encoded; a result of 65520 or more (the midpoint above 65504) is infinity. */
static uint16_t f32_to_f16_rne(float v) {
    uint32_t u;
    memcpy(&u, &v, sizeof u);
    const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (v != v) return (uint16_t)(sign | 0x7e00u);
    const double a = fabs((double)v);
    if (a >= 65520.0) return (uint16_t)(sign | 0x7c00u);
    int e;
    frexp(a, &e); /* a = m 2^e, m in [0.5, 1) */
    int unit_exp = e - 11;            /* 11 significant bits */
    if (unit_exp < -24) unit_exp = -24; /* subnormal spacing */
    const double q = ldexp(a, -unit_exp);
    double r = floor(q);
    const double frac = q - r;
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
    /* r units of 2^unit_exp; re-encode (r may have carried into the next binade) */
    const double val = ldexp(r, unit_exp);
    if (val == 0.0) return sign;
    int e2;
    frexp(val, &e2);
    const int E = e2 - 1 + 15; /* biased exponent of val = 1.f * 2^(e2-1) */
    if (E <= 0) return (uint16_t)(sign | (uint16_t)ldexp(val, 24)); /* subnormal */
    const uint16_t frac_bits = (uint16_t)(ldexp(val, -(e2 - 1)) * 1024.0 - 1024.0);
    return (uint16_t)(sign | (uint16_t)(E << 10) | frac_bits);
}

void orc_f32_to_f16(const float* in, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = f32_to_f16_rne(in[i]);
}

static float widen(const void* p, int64_t i, int dtype) {
    if (dtype == 1) return bf16_to_f32(((const uint16_t*)p)[i]);
    if (dtype == 2) return f16_to_f32(((const uint16_t*)p)[i]);
    return ((const float*)p)[i];
}

/* [moshi] dequantize_affine with scales and biases of any of the three types: w = s * c, then
 * + b, both in float32 (two roundings as written: with float32 scales the product is not always
 * exact). out float32 [rows, cols]. */
int orc_dequantize_typed(const uint32_t* packed, const void* scales, const void* biases, int sb_dtype,
                         int64_t rows, int64_t cols, int64_t group, int bits, float* out) {
    if (rows < 0 || sb_dtype < 0 || sb_dtype > 2 || !valid_params(cols, group, bits)) return -1;
    const int64_t words = cols * bits / 32, groups = cols / group;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            const uint32_t code = code_at(packed + r * words, c, bits);
            const float s = widen(scales, r * groups + c / group, sb_dtype);
            const float b = widen(biases, r * groups + c / group, sb_dtype);
            const float prod = s * (float)code;
            out[r * cols + c] = prod + b;
        }
    return 0;
}

/* [nuvec] quantized_matmul (transpose) with x and the scales and biases of any of the three types:
 * y[m, n] = sum_k x[m, k] w[n, k] in double, w as orc_dequantize_typed forms it. */
int orc_qmm_typed(const void* x, int x_dtype, int64_t m, const uint32_t* packed, const void* scales,
                  const void* biases, int sb_dtype, int64_t n, int64_t k, int64_t group, int bits, double* out) {
    if (m < 0 || n < 0 || x_dtype < 0 || x_dtype > 2) return -1;
    float* w = (float*)malloc(sizeof(float) * (size_t)(n * k > 0 ? n * k : 1));
    if (!w) return -2;
    const int rc = orc_dequantize_typed(packed, scales, biases, sb_dtype, n, k, group, bits, w);
    if (rc != 0) { free(w); return rc; }
    for (int64_t mm = 0; mm < m; ++mm)
        for (int64_t nn = 0; nn < n; ++nn) {
            double acc = 0.0;
            for (int64_t kk = 0; kk < k; ++kk) acc += (double)widen(x, mm * k + kk, x_dtype) * (double)w[nn * k + kk];
            out[mm * n + nn] = acc;
        }
    free(w);
    return 0;
}

/* [nuvec] quantized_matmul without the transpose, x and the scales and biases of any of the three
 * types: y[m, n] = sum over k of x[m, k] * w[k, n] in double, sequentially in k, for a weight stored
 * [k, n] whose rows orc_dequantize_typed forms (k rows of n values). */
int orc_qmm_nt_typed(const void* x, int x_dtype, int64_t m, const uint32_t* packed, const void* scales,
                     const void* biases, int sb_dtype, int64_t k, int64_t n, int64_t group, int bits, double* out) {
    if (m < 0 || k < 0 || x_dtype < 0 || x_dtype > 2) return -1;
    float* w = (float*)malloc(sizeof(float) * (size_t)(k * n > 0 ? k * n : 1));
    if (!w) return -2;
    const int rc = orc_dequantize_typed(packed, scales, biases, sb_dtype, k, n, group, bits, w);
    if (rc != 0) { free(w); return rc; }
    for (int64_t mm = 0; mm < m; ++mm)
        for (int64_t nn = 0; nn < n; ++nn) {
            double acc = 0.0;
            for (int64_t kk = 0; kk < k; ++kk) acc += (double)widen(x, mm * k + kk, x_dtype) * (double)w[kk * n + nn];
            out[mm * n + nn] = acc;
        }
    free(w);
    return 0;
}

/* [nuvec] quantize (module documentation and `quantize`: float16, bfloat16 or float32 w; scales and
 * biases in w's dtype) with [moshi]'s bias: each group of G values of a row, in the pages' order:
 *   bias  = the group minimum; scale = (max - min) / (2^bits - 1): the statistics in float32 (w
 *           widened exactly), both stored in sb_dtype (float32 as is; bf16 or float16 rounded to
 *           nearest even). nuvec_core's rule is sb_dtype = w's dtype; orc_quantize stores bf16, the
 *           type every kernel here consumes;
 *   code  = round((w - bias) / scale) with the stored bias and scale, the value of the formula
 *           itself (no intermediate rounding of the difference or the quotient), rounded half away
 *           from zero (the Rust `round` of the page) and clamped to [0, 2^bits - 1]; a group whose
 *           stored scale is 0 (all values equal, or a range below the narrower type's least value)
 *           takes code 0, so it dequantizes to the bias.
 * For a positive scale, code c >= 0 is the rounded quotient exactly when
 *     (c - 1/2) * scale <= w - bias < (c + 1/2) * scale,
 * which is decided by the exact sign of w - bias - (c +- 1/2) * scale (each (c +- 1/2) * scale has
 * at most 9 + 24 significant bits, exact in double). A double estimate is stepped until both hold.
 * A stored scale or bias that is not finite (an input that is not, or a statistic past the
 * narrower type's range) leaves the codes unspecified. Codes are packed into the row's bit stream
 * one bit at a time (orc_pack_codes). Returns 0, or -1 for parameters outside the format. */
static double quantize_code(float w, float bias, float scale, double top) {
    if (scale == 0.0f) return 0.0;
    double c = floor(((double)w - (double)bias) / (double)scale + 0.5);
    if (!(c >= 0.0)) c = 0.0; /* also a NaN estimate */
    if (c > top + 1.0) c = top + 1.0;
    while (c > 0.0 && sign_of_sum3(w, -(double)bias, -(c - 0.5) * (double)scale) < 0) c -= 1.0;
    while (c <= top && sign_of_sum3(w, -(double)bias, -(c + 0.5) * (double)scale) >= 0) c += 1.0;
    return c > top ? top : c;
}

/* v stored as dtype (float32 as is, bf16 / float16 rounded to nearest even) and read back. */
static float store_typed(void* p, int64_t i, int dtype, float v) {
    if (dtype == 1) {
        ((uint16_t*)p)[i] = f32_to_bf16_rne(v);
        return bf16_to_f32(((uint16_t*)p)[i]);
    }
    if (dtype == 2) {
        ((uint16_t*)p)[i] = f32_to_f16_rne(v);
        return f16_to_f32(((uint16_t*)p)[i]);
    }
    ((float*)p)[i] = v;
    return v;
}

int orc_quantize_typed(const void* w, int w_dtype, int64_t rows, int64_t cols, int64_t group, int bits,
                       uint32_t* packed, void* scales, void* biases, int sb_dtype) {
    if (rows < 0 || bits > 8 || group > 128 || !valid_params(cols, group, bits)) return -1;
    if (w_dtype < 0 || w_dtype > 2 || sb_dtype < 0 || sb_dtype > 2) return -1;
    uint8_t* codes = (uint8_t*)malloc((size_t)(rows * cols > 0 ? rows * cols : 1));
    if (!codes) return -2;
    const float top = (float)((1 << bits) - 1);
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t g = 0; g < cols / group; ++g) {
            float v[128];
            for (int64_t j = 0; j < group; ++j) v[j] = widen(w, r * cols + g * group + j, w_dtype);
            float lo = v[0], hi = v[0];
            for (int64_t j = 1; j < group; ++j) {
                if (v[j] < lo) lo = v[j];
                if (v[j] > hi) hi = v[j];
            }
            const float range = hi - lo;
            const int64_t gi = r * (cols / group) + g;
            const float sc = store_typed(scales, gi, sb_dtype, range / top);
            const float bi = store_typed(biases, gi, sb_dtype, lo);
            for (int64_t j = 0; j < group; ++j)
                codes[r * cols + g * group + j] = (uint8_t)quantize_code(v[j], bi, sc, (double)top);
        }
    const int rc = orc_pack_codes(codes, rows, cols, bits, packed);
    free(codes);
    return rc;
}

/* orc_quantize_typed with float32 or bf16 w and bf16 scales and biases. */
int orc_quantize(const void* w, int w_is_bf16, int64_t rows, int64_t cols, int64_t group, int bits,
                 uint32_t* packed, uint16_t* scales, uint16_t* biases) {
    return orc_quantize_typed(w, w_is_bf16 ? 1 : 0, rows, cols, group, bits, packed, scales, biases, 1);
}

/* [nuvec] gather_qmm (transpose form) with x and the scales and biases of any of the three types:
 * output batch i is orc_qmm_typed of x batch lhs[i] against weight batch rhs[i] (each defaulting
 * to i when null); an index past its operand gives a NaN batch. x [x_batches, m, k], packed
 * [w_batches, n, k*bits/32], scales/biases [w_batches, n, k/group]; out double [batch, m, n]. */
int orc_gather_qmm_typed(const void* x, int x_dtype, int64_t x_batches, int64_t m, const uint32_t* packed,
                         const void* scales, const void* biases, int sb_dtype, int64_t w_batches, int64_t n,
                         int64_t k, int64_t group, int bits, const uint32_t* lhs, const uint32_t* rhs,
                         int64_t batch, double* out) {
    if (batch < 0 || m < 0 || n < 0 || x_dtype < 0 || x_dtype > 2 || sb_dtype < 0 || sb_dtype > 2) return -1;
    if (!valid_params(k, group, bits)) return -1;
    const int64_t xsize = x_dtype == 0 ? 4 : 2, sbsize = sb_dtype == 0 ? 4 : 2;
    const int64_t words = k * bits / 32, groups = k / group;
    for (int64_t i = 0; i < batch; ++i) {
        const int64_t li = lhs ? (int64_t)lhs[i] : i;
        const int64_t ri = rhs ? (int64_t)rhs[i] : i;
        double* yi = out + i * m * n;
        if (li >= x_batches || ri >= w_batches) {
            for (int64_t t = 0; t < m * n; ++t) yi[t] = NAN;
            continue;
        }
        const int rc = orc_qmm_typed((const uint8_t*)x + li * m * k * xsize, x_dtype, m, packed + ri * n * words,
                                     (const uint8_t*)scales + ri * n * groups * sbsize,
                                     (const uint8_t*)biases + ri * n * groups * sbsize, sb_dtype, n, k, group,
                                     bits, yi);
        if (rc != 0) return rc;
    }
    return 0;
}
