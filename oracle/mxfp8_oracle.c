/*
 * MXFP8 block quantization: the CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow definition that the
 * GPU path is checked against.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it.  It shares no code, header, table
 * or constant with the HIP library, and the HIP library never calls it.
 *
 * What is computed, and where it is stated:
 *   - Blocks hold 32 elements (Megatron-Core quantized_dbuffer page, "Data",
 *     _MXFP8_BLOCK_SIZE).  A rowwise block is 32 consecutive elements of one
 *     row; its scales form a [rows, cols/32] array (Mojo
 *     DistributedAllGatherRMSNormQuantMXFP8 page, "Args", outputs_scale).  A
 *     columnwise block is 32 consecutive rows of one column, so one columnwise
 *     scale row covers a 32-row block (quantized_dbuffer page, API,
 *     _block_atomic_to_flat); its scales form a [rows/32, cols] array.
 *   - Elements are float8_e4m3fn and scales float8_e8m0fnu (Mojo page,
 *     "Parameters", quant_dtype and scales_dtype).
 *   - Both data planes share one [rows, cols] layout (quantized_dbuffer page,
 *     Functions: _rowwise_scale_layout / _columnwise_scale_layout); storage is
 *     compact and unswizzled (API: QuantizedDBuffer, get_tensor_view).
 *   - The pages do not state the scale rule or the rounding.  This oracle takes
 *     the OCP Microscaling (MX) v1.0 convention: the block scale is
 *     2^(floor(log2 amax) - 8), where 8 is the exponent of e4m3's largest
 *     normal (448 = 1.75 * 2^8); an all-zero block gets the smallest scale
 *     (byte 0x00); elements are rounded to nearest, ties to even, and
 *     saturate at +-448.  Further readings where the pages are silent:
 *     a scale below 2^-127 is clamped to byte 0x00; a block holding a NaN or
 *     an infinity gets scale byte 0xFF and every element byte sign|0x7F; the
 *     sign of zero is kept.
 *   - A float32 master weight (quantized_dbuffer page, QuantizedDBuffer.quantize_
 *     on a local master shard) follows the same rule on its float32 values.
 *   - RMSNorm (Mojo page, "Args": gammas, float32 epsilons, weight_offsets):
 *     y = x / sqrt(mean(x^2) + eps) * (gamma + offset), rounded once to bf16;
 *     the quantized copy is a plain rowwise quantize of that bf16 (Mojo page,
 *     execute: the quantize reads the same bf16 that is written as normed).
 *
 * All floating-point work is in double precision; every scaling is by a power
 * of two and therefore exact.  Parallelism (OpenMP) is over independent rows
 * or row strips only; no arithmetic is reordered.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define MX_BLOCK 32
#define E4M3_MAX 448.0 /* 1.75 * 2^8, the largest finite float8_e4m3fn */
#define E4M3_EMAX 8    /* exponent of E4M3_MAX */
#define E8M0_BIAS 127

/* bf16 is the upper half of an IEEE binary32. */
static double bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* floor(log2(a)) for finite a > 0. */
static int floor_log2(double a) {
    int e;
    frexp(a, &e); /* a = f * 2^e with f in [0.5, 1) */
    return e - 1;
}

/* Round a non-negative value to the nearest multiple of q (a power of two),
 * ties to the even multiple.  a / q is exact, so this is exact. */
static double round_half_even_to(double a, double q) {
    double t = a / q;
    double m = floor(t);
    double frac = t - m;
    if (frac > 0.5 || (frac == 0.5 && fmod(m, 2.0) == 1.0)) m += 1.0;
    return m * q;
}

/* E8M0 scale byte of one block of n values. */
static int block_scale_byte(const double *v, int n) {
    double amax = 0.0;
    for (int i = 0; i < n; ++i) {
        if (!isfinite(v[i])) return 0xFF;
        double a = fabs(v[i]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0) return 0x00;
    int s = floor_log2(amax) - E4M3_EMAX + E8M0_BIAS;
    if (s < 0) s = 0;
    if (s > 254) s = 254;
    return s;
}

/* float8_e4m3fn byte of v: round to nearest even, saturate at +-448.
 * e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent
 * field 0 holds subnormals m * 2^-9; 0x7F / 0xFF are NaN; no infinities. */
static uint8_t e4m3_byte(double v) {
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    if (a >= E4M3_MAX) return sign | 0x7E;
    if (a == 0.0) return sign;
    int e = floor_log2(a);
    if (e < -6) e = -6;                       /* below 2^-6 the grid is 2^-9 */
    double r = round_half_even_to(a, ldexp(1.0, e - 3));
    if (r == 0.0) return sign;
    int er = floor_log2(r);                   /* r may have moved up a binade */
    if (er < -6) return sign | (uint8_t)(r / ldexp(1.0, -9));
    int mant = (int)((r / ldexp(1.0, er) - 1.0) * 8.0);
    return sign | (uint8_t)(((er + 7) << 3) | mant);
}

/* Quantize one block of n values v[0..n-1]; element bytes go to q, stride
 * apart, and the scale byte to *s. */
static void quantize_values(const double *v, int n, uint8_t *q, int64_t stride,
                            uint8_t *s) {
    int sb = block_scale_byte(v, n);
    *s = (uint8_t)sb;
    for (int i = 0; i < n; ++i) {
        uint8_t b;
        if (sb == 0xFF)
            b = (signbit(v[i]) ? 0x80 : 0x00) | 0x7F;
        else
            b = e4m3_byte(ldexp(v[i], E8M0_BIAS - sb));
        q[(int64_t)i * stride] = b;
    }
}

/* One block of bf16 values, stride apart in x (and in q). */
static void quantize_block(const uint16_t *x, int64_t stride, int n,
                           uint8_t *q, uint8_t *s) {
    double v[MX_BLOCK];
    for (int i = 0; i < n; ++i) v[i] = bf16_value(x[(int64_t)i * stride]);
    quantize_values(v, n, q, stride, s);
}

/* One block of float32 values (a float32 master weight), stride apart. */
static void quantize_block_f32(const float *x, int64_t stride, int n,
                               uint8_t *q, uint8_t *s) {
    double v[MX_BLOCK];
    for (int i = 0; i < n; ++i) v[i] = (double)x[(int64_t)i * stride];
    quantize_values(v, n, q, stride, s);
}

/* Rowwise plane: q[r, c] and s[r, c/32] from x[r, 32j .. 32j+31]. */
void mxfp8_oracle_quantize_rowwise(const uint16_t *x, int64_t rows, int64_t cols,
                                   uint8_t *q, uint8_t *s) {
    int64_t nb = cols / MX_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < nb; ++j)
            quantize_block(x + r * cols + j * MX_BLOCK, 1, MX_BLOCK,
                           q + r * cols + j * MX_BLOCK, s + r * nb + j);
}

/* Columnwise plane: q[r, c] (same layout as x) and s[r/32, c] from
 * x[32i .. 32i+31, c]. */
void mxfp8_oracle_quantize_colwise(const uint16_t *x, int64_t rows, int64_t cols,
                                   uint8_t *q, uint8_t *s) {
    int64_t nb = rows / MX_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nb; ++i)
        for (int64_t c = 0; c < cols; ++c)
            quantize_block(x + i * MX_BLOCK * cols + c, cols, MX_BLOCK,
                           q + i * MX_BLOCK * cols + c, s + i * cols + c);
}

/* The same two planes of a float32 tensor. */
void mxfp8_oracle_quantize_rowwise_f32(const float *x, int64_t rows, int64_t cols,
                                       uint8_t *q, uint8_t *s) {
    int64_t nb = cols / MX_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < nb; ++j)
            quantize_block_f32(x + r * cols + j * MX_BLOCK, 1, MX_BLOCK,
                               q + r * cols + j * MX_BLOCK, s + r * nb + j);
}

void mxfp8_oracle_quantize_colwise_f32(const float *x, int64_t rows, int64_t cols,
                                       uint8_t *q, uint8_t *s) {
    int64_t nb = rows / MX_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nb; ++i)
        for (int64_t c = 0; c < cols; ++c)
            quantize_block_f32(x + i * MX_BLOCK * cols + c, cols, MX_BLOCK,
                               q + i * MX_BLOCK * cols + c, s + i * cols + c);
}

/* Value of one float8_e4m3fn byte (NaN for 0x7F / 0xFF). */
static double e4m3_value(uint8_t b) {
    int sign = b >> 7, ef = (b >> 3) & 0xF, m = b & 0x7;
    double a;
    if (ef == 0xF && m == 0x7) return NAN;
    if (ef == 0)
        a = ldexp((double)m, -9);
    else
        a = ldexp(1.0 + m / 8.0, ef - 7);
    return sign ? -a : a;
}

/* Value of one float8_e8m0fnu byte: 2^(b - 127), NaN for 0xFF. */
static double e8m0_value(uint8_t b) {
    return b == 0xFF ? NAN : ldexp(1.0, (int)b - E8M0_BIAS);
}

/* Dequantize to exact doubles.  axis 0: s is [rows, cols/32] (rowwise);
 * axis 1: s is [rows/32, cols] (columnwise). */
void mxfp8_oracle_dequantize(const uint8_t *q, const uint8_t *s, int64_t rows,
                             int64_t cols, int axis, double *out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            uint8_t sb = axis == 0 ? s[r * (cols / MX_BLOCK) + c / MX_BLOCK]
                                   : s[(r / MX_BLOCK) * cols + c];
            out[r * cols + c] = e4m3_value(q[r * cols + c]) * e8m0_value(sb);
        }
}

/* One entry of the MXFP8 matrix product: sum over k of the exact values of
 * A[m, k] and B[n, k], both given as rowwise planes (scales one per 32 k).
 * *abs_sum receives the sum of |A[m, k] * B[n, k]| (for error bounds). */
static double gemm_entry(const uint8_t *qa, const uint8_t *sa, const uint8_t *qb,
                         const uint8_t *sb, int64_t K, int64_t m, int64_t n,
                         double *abs_sum) {
    double acc = 0.0, mag = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double a = e4m3_value(qa[m * K + k]) * e8m0_value(sa[m * (K / MX_BLOCK) + k / MX_BLOCK]);
        double b = e4m3_value(qb[n * K + k]) * e8m0_value(sb[n * (K / MX_BLOCK) + k / MX_BLOCK]);
        acc += a * b;
        mag += fabs(a * b);
    }
    *abs_sum = mag;
    return acc;
}

/* out[m, n] = sum_k A[m, k] * B[n, k] for A [M, K] and B [N, K] in MXFP8
 * rowwise planes (the product a linear layer computes from a quantized
 * activation and a quantized weight: quantization.utils page, mm_mxfp8). */
void mxfp8_oracle_gemm(const uint8_t *qa, const uint8_t *sa, const uint8_t *qb,
                       const uint8_t *sb, int64_t M, int64_t N, int64_t K,
                       double *out, double *abs_sum) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            out[m * N + n] = gemm_entry(qa, sa, qb, sb, K, m, n, &abs_sum[m * N + n]);
}

/* The same product at count chosen positions (ms[i], ns[i]). */
void mxfp8_oracle_gemm_at(const uint8_t *qa, const uint8_t *sa, const uint8_t *qb,
                          const uint8_t *sb, int64_t K, const int64_t *ms,
                          const int64_t *ns, int64_t count, double *out,
                          double *abs_sum) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        out[i] = gemm_entry(qa, sa, qb, sb, K, ms[i], ns[i], &abs_sum[i]);
}

/* Round doubles to bf16 bit patterns: nearest, ties to even; NaN -> 0x7FC0
 * with the input's sign; overflow past the largest finite bf16 -> infinity. */
void mxfp8_oracle_round_bf16(const double *in, int64_t n, uint16_t *out) {
    for (int64_t i = 0; i < n; ++i) {
        double v = in[i];
        uint16_t sign = signbit(v) ? 0x8000 : 0x0000;
        double a = fabs(v);
        if (isnan(v)) { out[i] = sign | 0x7FC0; continue; }
        if (a == 0.0) { out[i] = sign; continue; }
        int e = isinf(a) ? 128 : floor_log2(a);
        if (e < -126) e = -126;               /* bf16 subnormals: grid 2^-133 */
        double r = isinf(a) ? a : round_half_even_to(a, ldexp(1.0, e - 7));
        if (r >= ldexp(1.0, 128)) { out[i] = sign | 0x7F80; continue; }
        if (r == 0.0) { out[i] = sign; continue; }
        int er = floor_log2(r);
        uint16_t bits;
        if (er < -126)
            bits = (uint16_t)(r / ldexp(1.0, -133));
        else
            bits = (uint16_t)(((er + 127) << 7) |
                              (int)((r / ldexp(1.0, er) - 1.0) * 128.0));
        out[i] = sign | bits;
    }
}

/* 1 / sqrt(mean(x_row^2) + eps), the row's reciprocal RMS. */
static double row_rstd(const uint16_t *x_row, int64_t cols, float eps) {
    double ss = 0.0;
    for (int64_t c = 0; c < cols; ++c) {
        double v = bf16_value(x_row[c]);
        ss += v * v;
    }
    return 1.0 / sqrt(ss / (double)cols + (double)eps);
}

/* RMSNorm of each row before the final rounding, in double:
 * y[r, c] = x[r, c] / sqrt(mean_c(x[r, :]^2) + eps) * (gamma[c] + offset). */
void mxfp8_oracle_rmsnorm_f64(const uint16_t *x, const uint16_t *gamma,
                              float weight_offset, float eps, int64_t rows,
                              int64_t cols, double *y) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double rstd = row_rstd(x + r * cols, cols, eps);
        for (int64_t c = 0; c < cols; ++c)
            y[r * cols + c] = bf16_value(x[r * cols + c]) * rstd *
                              (bf16_value(gamma[c]) + (double)weight_offset);
    }
}

/* RMSNorm rounded once to bf16 (the "normed" output). */
void mxfp8_oracle_rmsnorm(const uint16_t *x, const uint16_t *gamma,
                          float weight_offset, float eps, int64_t rows,
                          int64_t cols, uint16_t *normed) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double rstd = row_rstd(x + r * cols, cols, eps);
        for (int64_t c = 0; c < cols; ++c) {
            double y = bf16_value(x[r * cols + c]) * rstd *
                       (bf16_value(gamma[c]) + (double)weight_offset);
            mxfp8_oracle_round_bf16(&y, 1, &normed[r * cols + c]);
        }
    }
}

/* Fused op: normed = RMSNorm(x) in bf16, then the rowwise plane of normed. */
void mxfp8_oracle_rmsnorm_quantize(const uint16_t *x, const uint16_t *gamma,
                                   float weight_offset, float eps, int64_t rows,
                                   int64_t cols, uint16_t *normed, uint8_t *q,
                                   uint8_t *s) {
    mxfp8_oracle_rmsnorm(x, gamma, weight_offset, eps, rows, cols, normed);
    mxfp8_oracle_quantize_rowwise(normed, rows, cols, q, s);
}

void mxfp8_oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int mxfp8_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
