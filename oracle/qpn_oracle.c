/*
 * qpn_oracle.c -- plain, slow, FP64 CPU oracle for the QPN weight-streaming
 * skinny GEMM (NVFP4 and FP8 weights times FP16 activations).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * CPU-baseline leg of the benchmark may load or call this library.  It shares
 * no code, header, table or constant with the HIP library; the two are
 * compared, never combined.
 *
 * Sources.  The method is described on three web pages:
 *   [P1] taozi.news, "四张 2017 年 V100 跑通 Qwen 3 NVFP4 推理，性能追平 RTX 5090"
 *   [P2] aiwitness.kr, "VOLTA에서 NVFP4 구동! Blackwell용으로 설계되었지만 ..."
 *   [P3] lcz.me, "前情提要 整台洋垃圾V100 16G雙卡"
 * [P1 section "自研 QPN 内核"] and [P2 section "내가 실제로 만든 것"] state the
 * problem: weights stay in their published compressed format (NVFP4 for the
 * FP4 regions, FP8 for the FP8 regions) and are multiplied by FP16
 * activations of 1..8 rows, with no separate dequantize-to-FP16 pass.
 * [P3, table of NVFP4 support on sm_70] names the NVFP4 element and scale
 * formats: E2M1 codes and UE4M3 scales.  The pages print no bit layout, no
 * block size and no rounding rule; the readings taken here are:
 *   - E2M1 and E4M3 are the OCP formats (OCP Microscaling Formats v1.0 for
 *     FP4 E2M1; OCP 8-bit Floating Point for E4M3, the "FN" variant with
 *     bias 7, max 448, NaN = S.1111.111 and no infinities).
 *   - UE4M3 is E4M3 without the sign bit; only bytes 0x00..0x7E are valid.
 *   - NVFP4: 16-element blocks along K, one UE4M3 scale per block, one FP32
 *     tensor scale g = amax / (6 * 448).
 *   - FP8: one FP32 scale per output channel, s = row amax / 448.
 *   - Rounding is round-to-nearest, ties to the even code, saturating at the
 *     largest finite value ("pure round" in [P3, quantisation option table]).
 *   - The code's sign bit is the IEEE sign bit of the value being narrowed;
 *     a NaN input (only 0/0 in degenerate blocks) narrows to code 0.
 *
 * Every floating-point step of the pack is one FP32 IEEE round-to-nearest
 * operation in the order written here; build with -ffp-contract=off.  All
 * decoding, dequantisation and the GEMM itself run in FP64.
 *
 * Parity pins for every function live under tests/ (exhaustive format
 * tables, library conversions, hand-worked examples, exact rational dot
 * products); see the function comments for which pin covers what.
 */
#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------------- */
/* Element formats, decoded to FP64 straight from their bit definitions.      */
/* ------------------------------------------------------------------------- */

/* FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; no Inf/NaN.
 * Exponent field 0 is subnormal: 0.5 * m.  Pinned exhaustively against the
 * OCP table (tests/golden/e2m1_values.txt). */
ORACLE_API double qpn_oracle_e2m1_value(int code)
{
    int s = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int m = code & 1;
    double mag = (e == 0) ? 0.5 * (double)m
                          : ldexp(1.0 + 0.5 * (double)m, e - 1);
    return s ? -mag : mag;
}

/* FP8 E4M3 ("FN"): 1 sign, 4 exponent (bias 7), 3 mantissa bits.  The
 * all-ones exponent with all-ones mantissa is NaN; there are no infinities.
 * Exponent field 0 is subnormal: m * 2^-9.  Pinned against torch's
 * float8_e4m3fn decode of all 256 bytes and the OCP landmarks. */
ORACLE_API double qpn_oracle_e4m3_value(int code)
{
    int s = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* UE4M3 block scale: the magnitude half of E4M3.  Valid bytes are
 * 0x00..0x7E; anything else (0x7F is NaN, 0x80.. carry a sign bit) is
 * rejected with -1. */
ORACLE_API int qpn_oracle_ue4m3_value(int byte, double *out)
{
    if (byte < 0 || byte > 0x7E)
        return -1;
    *out = qpn_oracle_e4m3_value(byte);
    return 0;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits. */
ORACLE_API double qpn_oracle_f16_value(uint16_t h)
{
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double mag;
    if (e == 31)
        mag = f ? NAN : INFINITY;
    else if (e == 0)
        mag = ldexp((double)f, -24);
    else
        mag = ldexp(1.0 + (double)f / 1024.0, e - 15);
    return s ? -mag : mag;
}

/* FP64 -> binary16, round to nearest, ties to even, overflow to +-Inf.
 * Pinned against numpy's float64 -> float16 conversion. */
ORACLE_API uint16_t qpn_oracle_f16_round(double v)
{
    uint16_t s;
    double a, q;
    int e, E;
    if (isnan(v))
        return 0x7E00;
    s = signbit(v) ? 0x8000 : 0;
    a = fabs(v);
    if (isinf(a))
        return s | 0x7C00;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: multiples of 2^-24; a * 2^24 is exact */
        q = nearbyint(ldexp(a, 24));
        return s | (uint16_t)q; /* q == 1024 is the smallest normal */
    }
    frexp(a, &e); /* a = f * 2^e with f in [0.5, 1) */
    E = e - 1;    /* a in [2^E, 2^(E+1)) */
    q = nearbyint(ldexp(a, 10 - E)); /* 11-bit significand in [1024, 2048] */
    if (q == 2048.0) {
        q = 1024.0;
        E += 1;
    }
    if (E > 15)
        return s | 0x7C00;
    return (uint16_t)(s | (uint16_t)((E + 15) << 10) | (uint16_t)(q - 1024.0));
}

/* ------------------------------------------------------------------------- */
/* Narrowing quantisers (FP32 in, code out).                                  */
/* ------------------------------------------------------------------------- */

/* Sorted non-negative value tables, built from the decoders above.  For both
 * formats the code of a non-negative value is its index in this table (codes
 * increase with value); tests pin that monotonicity. */
static double e2m1_pos[8];
static double e4m3_pos[127]; /* codes 0x00..0x7E */
static int tables_ready = 0;

static void build_tables(void)
{
    int i;
    if (tables_ready)
        return;
    for (i = 0; i < 8; ++i)
        e2m1_pos[i] = qpn_oracle_e2m1_value(i);
    for (i = 0; i < 127; ++i)
        e4m3_pos[i] = qpn_oracle_e4m3_value(i);
    tables_ready = 1;
}

/* Index of the table value nearest to a (a >= 0, finite): values at or above
 * the top saturate to it; an exact midpoint goes to the even index. */
static int nearest_index(double a, const double *v, int n)
{
    int lo = 0, hi = n - 1, mid;
    double midpoint;
    if (a >= v[n - 1])
        return n - 1;
    /* invariant: v[lo] <= a < v[hi] */
    while (hi - lo > 1) {
        mid = (lo + hi) / 2;
        if (v[mid] <= a)
            lo = mid;
        else
            hi = mid;
    }
    midpoint = 0.5 * (v[lo] + v[hi]); /* exact: both are short dyadics */
    if (a < midpoint)
        return lo;
    if (a > midpoint)
        return hi;
    return (lo % 2 == 0) ? lo : hi;
}

/* FP32 -> E2M1 code, nearest-even, saturating at +-6. */
ORACLE_API int qpn_oracle_quant_e2m1(float t)
{
    int idx;
    build_tables();
    if (isnan(t))
        return 0;
    idx = nearest_index(fabs((double)t), e2m1_pos, 8);
    return signbit(t) ? (idx | 0x8) : idx;
}

/* FP32 -> E4M3 code, nearest-even, saturating at +-448 (never NaN). */
ORACLE_API int qpn_oracle_quant_e4m3(float t)
{
    int idx;
    build_tables();
    if (isnan(t))
        return 0;
    idx = nearest_index(fabs((double)t), e4m3_pos, 127);
    return signbit(t) ? (idx | 0x80) : idx;
}

/* ------------------------------------------------------------------------- */
/* Pack: the quantisation recipes, FP32 step by step.                        */
/* ------------------------------------------------------------------------- */

/* NVFP4 tensor scale.  amax = max |w| over the whole tensor (exact);
 * g = amax / 2688 with 2688 = 6 * 448 (largest E2M1 value times largest
 * UE4M3 value), one FP32 division. */
ORACLE_API float qpn_oracle_nvfp4_tensor_scale(const float *w, int64_t count,
                                               float *amax_out)
{
    float amax = 0.0f, a;
    int64_t i;
    for (i = 0; i < count; ++i) {
        a = fabsf(w[i]);
        if (a > amax)
            amax = a;
    }
    if (amax_out)
        *amax_out = amax;
    return amax / 2688.0f;
}

/* NVFP4 pack of `rows` rows of length k (k % 16 == 0) with tensor scale g.
 * Output is the canonical, unpermuted form:
 *   codes  [rows, k/2]  element 2j in the low nibble of byte j, 2j+1 high;
 *   scales [rows, k/16] one UE4M3 byte per 16-element block.
 * Per block:  a = max|w| (exact);  if g == 0 the scale is 0, else
 *   r = (a / 6) / g   (two FP32 divisions)   and   sc = E4M3 code of r.
 * S = value of sc.  If S == 0 every code is 0; else d = S * g (FP32) and
 *   each code is the E2M1 code of w / d (FP32 division). */
ORACLE_API int qpn_oracle_pack_nvfp4_rows(const float *w, int64_t rows,
                                          int64_t k, float g,
                                          uint8_t *codes, uint8_t *scales)
{
    int64_t r;
    if (k % 16 != 0 || rows < 0 || k < 0)
        return -1;
    build_tables();
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        int64_t b;
        for (b = 0; b < k / 16; ++b) {
            const float *blk = w + r * k + b * 16;
            float a = 0.0f, ratio, S, d, t;
            int sc, i, q[16];
            for (i = 0; i < 16; ++i)
                if (fabsf(blk[i]) > a)
                    a = fabsf(blk[i]);
            if (g == 0.0f) {
                sc = 0;
            } else {
                ratio = a / 6.0f;
                ratio = ratio / g;
                sc = qpn_oracle_quant_e4m3(ratio);
            }
            scales[r * (k / 16) + b] = (uint8_t)sc;
            S = (float)qpn_oracle_e4m3_value(sc); /* exact in FP32 */
            for (i = 0; i < 16; ++i) {
                if (S == 0.0f) {
                    q[i] = 0;
                } else {
                    d = S * g;
                    t = blk[i] / d;
                    q[i] = qpn_oracle_quant_e2m1(t);
                }
            }
            for (i = 0; i < 8; ++i)
                codes[r * (k / 2) + b * 8 + i] =
                    (uint8_t)(q[2 * i] | (q[2 * i + 1] << 4));
        }
    }
    return 0;
}

/* FP8 pack of `rows` rows of length k.  Per row:  a = max|w| (exact);
 * s = a / 448 (FP32) is the stored row scale.  If s == 0 every code is 0;
 * else each code is the E4M3 code of w / s (FP32 division).
 * codes [rows, k] one byte per element; row_scale [rows]. */
ORACLE_API int qpn_oracle_pack_fp8_rows(const float *w, int64_t rows,
                                        int64_t k, uint8_t *codes,
                                        float *row_scale)
{
    int64_t r;
    if (rows < 0 || k < 0)
        return -1;
    build_tables();
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        const float *row = w + r * k;
        float a = 0.0f, s, t;
        int64_t i;
        for (i = 0; i < k; ++i)
            if (fabsf(row[i]) > a)
                a = fabsf(row[i]);
        s = a / 448.0f;
        row_scale[r] = s;
        for (i = 0; i < k; ++i) {
            if (s == 0.0f) {
                codes[r * k + i] = 0;
            } else {
                t = row[i] / s;
                codes[r * k + i] = (uint8_t)qpn_oracle_quant_e4m3(t);
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Dequantisation (exact in FP64) and the GEMM.                              */
/* ------------------------------------------------------------------------- */

/* w_hat[r, i] = E2M1(code) * UE4M3(scale of its block) * g, exact in FP64
 * (at most 2 + 4 + 24 significant bits).  Returns -1 on an invalid scale. */
ORACLE_API int qpn_oracle_dequant_nvfp4(const uint8_t *codes,
                                        const uint8_t *scales, float g,
                                        int64_t rows, int64_t k, double *w_hat)
{
    int64_t r, i;
    for (r = 0; r < rows; ++r) {
        for (i = 0; i < k; ++i) {
            uint8_t byte = codes[r * (k / 2) + i / 2];
            int code = (i % 2 == 0) ? (byte & 0xF) : (byte >> 4);
            double S;
            if (qpn_oracle_ue4m3_value(scales[r * (k / 16) + i / 16], &S) != 0)
                return -1;
            w_hat[r * k + i] = qpn_oracle_e2m1_value(code) * S * (double)g;
        }
    }
    return 0;
}

/* w_hat[r, i] = E4M3(code) * s_r, exact in FP64. */
ORACLE_API void qpn_oracle_dequant_fp8(const uint8_t *codes,
                                       const float *row_scale, int64_t rows,
                                       int64_t k, double *w_hat)
{
    int64_t r, i;
    for (r = 0; r < rows; ++r)
        for (i = 0; i < k; ++i)
            w_hat[r * k + i] =
                qpn_oracle_e4m3_value(codes[r * k + i]) * (double)row_scale[r];
}

/* The plain definition of the product: y[mi, r] = sum_i x[mi, i] * w_hat[r, i]
 * with x the FP16 activations [m, k] (bit patterns) and w_hat [rows, k] in
 * FP64; naive loops, natural k order, one FP64 accumulator per output.
 * Parallel over output channels only, so the result is independent of the
 * thread count. */
ORACLE_API void qpn_oracle_gemm_f64(const double *w_hat, const uint16_t *x,
                                    int m, int64_t rows, int64_t k, double *y)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        int mi;
        int64_t i;
        for (mi = 0; mi < m; ++mi) {
            double acc = 0.0;
            for (i = 0; i < k; ++i)
                acc += qpn_oracle_f16_value(x[(int64_t)mi * k + i]) *
                       w_hat[r * k + i];
            y[(int64_t)mi * rows + r] = acc;
        }
    }
}

/* NVFP4 GEMM straight from the canonical codes and scales: each weight is
 * decoded as it is used (no dequantised copy), the FP64 product summed in
 * natural k order.  y is [m, rows].  Returns -1 on an invalid scale byte. */
ORACLE_API int qpn_oracle_gemm_nvfp4(const uint8_t *codes,
                                     const uint8_t *scales, float g,
                                     const uint16_t *x, int m, int64_t rows,
                                     int64_t k, double *y)
{
    int64_t r;
    int bad = 0;
    if (k % 16 != 0)
        return -1;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (r = 0; r < rows; ++r) {
        int mi;
        int64_t i;
        for (mi = 0; mi < m; ++mi) {
            double acc = 0.0;
            for (i = 0; i < k; ++i) {
                uint8_t byte = codes[r * (k / 2) + i / 2];
                int code = (i % 2 == 0) ? (byte & 0xF) : (byte >> 4);
                double S, wv;
                if (qpn_oracle_ue4m3_value(scales[r * (k / 16) + i / 16], &S)) {
                    bad = 1;
                    S = NAN;
                }
                wv = qpn_oracle_e2m1_value(code) * S * (double)g;
                acc += qpn_oracle_f16_value(x[(int64_t)mi * k + i]) * wv;
            }
            y[(int64_t)mi * rows + r] = acc;
        }
    }
    return bad ? -1 : 0;
}

/* FP8 GEMM straight from the codes: y[mi, r] = sum_i x * E4M3(code) * s_r. */
ORACLE_API void qpn_oracle_gemm_fp8(const uint8_t *codes,
                                    const float *row_scale, const uint16_t *x,
                                    int m, int64_t rows, int64_t k, double *y)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        int mi;
        int64_t i;
        for (mi = 0; mi < m; ++mi) {
            double acc = 0.0;
            for (i = 0; i < k; ++i) {
                double wv = qpn_oracle_e4m3_value(codes[r * k + i]) *
                            (double)row_scale[r];
                acc += qpn_oracle_f16_value(x[(int64_t)mi * k + i]) * wv;
            }
            y[(int64_t)mi * rows + r] = acc;
        }
    }
}

/* Greedy argmax over FP16 logits [m, n]: for each row, the lowest index whose
 * value equals the row maximum (values compared as numbers, so -0 == +0).
 * This is the selection the drafter fix in [P1 section
 * "一些工程细节与长上下文发现"] asks for: greedy / local argmax. */
ORACLE_API void qpn_oracle_argmax_f16(const uint16_t *logits, int m, int64_t n,
                                      int32_t *out)
{
    int mi;
    for (mi = 0; mi < m; ++mi) {
        int64_t j, best = 0;
        double bv = -INFINITY;
        for (j = 0; j < n; ++j) {
            double v = qpn_oracle_f16_value(logits[(int64_t)mi * n + j]);
            if (j == 0 || v > bv) {
                bv = v;
                best = j;
            }
        }
        out[mi] = (int32_t)best;
    }
}

/* Threads the OpenMP loops above run with (reported by the CPU baseline). */
ORACLE_API int qpn_oracle_threads(void) { return omp_get_max_threads(); }

/* Sets the threads of later parallel loops (the CPU baseline also times the
 * oracle on one thread).  Results do not depend on it: every loop is
 * parallel over output rows only. */
ORACLE_API void qpn_oracle_set_threads(int n)
{
    if (n >= 1)
        omp_set_num_threads(n);
}

/* Round an FP64 result array to FP16 bit patterns (the returned logits). */
ORACLE_API void qpn_oracle_round_f16_array(const double *y, int64_t count,
                                           uint16_t *out)
{
    int64_t i;
    for (i = 0; i < count; ++i)
        out[i] = qpn_oracle_f16_round(y[i]);
}
