/*
 * oracle.c -- CPU oracle for the MXFP4 W4A8 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the
 * cpu_baseline leg of bench.py; never by the library.  Shares no code with
 * the HIP path.  Page citations as in oracle.h ([P1], [P2], [P3]).
 *
 * Readings of points the pages leave open:
 *  R1  Block exponents are the exact-arithmetic values of the page's closed
 *      forms (floor(log2 amax)-2 and ceil(log2(amax/6))), i.e. the integers
 *      that satisfy the page's stated ranges [4,8) and (3,6]; not a float
 *      log2 that can land one off near a power of two.
 *  R2  The per-block squared error is summed in fp32, element order
 *      0..31, left to right, each square rounded to fp32 before the add.
 *  R3  mse: the finer exponent wins only on a strictly smaller error; when
 *      the no-clip exponent is already -127 the finer one has no e8m0 byte
 *      and is not tried.
 *  R4  The NVFP4 scale is divided by the global divisor with an IEEE
 *      (correctly rounded) fp32 division, then multiplied by the e2m1 value.
 *  R5  Per-token fp8: s = amax/448 (fp32 division), codes = RNE e4m3 of
 *      x/s (fp32 division), saturating at +-448, sign kept; s = 1 for an
 *      all-zero row.
 *  R6  GEMM reference: exact products, fp64 accumulation, token scale
 *      applied after the sum; not rounded to bf16.
 *
 * PARITY PINS: every function here is pinned by tests/test_oracle_*.py to
 * facts the pages or the mathematics fix (printed grid and rules, closed
 * forms, exhaustive or boundary sweeps, brute force on tiny inputs, library
 * casts).  Function with no external pin: none.
 */
#include "oracle.h"

#include <float.h>
#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* Threads of the parallel loops below (timing only: every loop writes disjoint
 * outputs, so no result depends on it). */
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int orc_max_threads(void) { return omp_get_max_threads(); }

/* [P1] module constants: the eight e2m1 magnitudes, index = low three bits. */
static const float E2M1_GRID[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

/* ------------------------------------------------------------------------ */
/* number formats                                                            */
/* ------------------------------------------------------------------------ */

/* [P1] unpack_e2m1: magnitude from the grid by code&7, negated when bit 3 is
 * set.  Code 8 is negative zero. */
float orc_e2m1_value(int code) {
    float mag = E2M1_GRID[code & 7];
    return (code & 8) ? -mag : mag;
}

/* OCP E4M3FN (the float8_e4m3fn type of the NVFP4 weight scale in [P1]
 * RadianceNvfp4ToMxfp4.create_weights): 1 sign, 4 exponent (bias 7),
 * 3 mantissa bits; exponent 0 is subnormal; 0x7F/0xFF are NaN; no inf. */
double orc_e4m3_value(uint8_t b) {
    int s = b >> 7, E = (b >> 3) & 15, m = b & 7;
    double v;
    if (E == 15 && m == 7) return NAN;
    if (E == 0)
        v = ldexp((double)m, -9);              /* m/8 * 2^(1-7) */
    else
        v = ldexp((double)(8 + m), E - 10);    /* (1+m/8) * 2^(E-7) */
    return s ? -v : v;
}

double orc_f16_value(uint16_t h) {
    int s = h >> 15, E = (h >> 10) & 31, m = h & 1023;
    double v;
    if (E == 31) return m ? NAN : (s ? -INFINITY : INFINITY);
    if (E == 0)
        v = ldexp((double)m, -24);
    else
        v = ldexp((double)(1024 + m), E - 25);
    return s ? -v : v;
}

float orc_bf16_value(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round a finite fp32 to the nearest E4M3FN value, ties to the even code,
 * saturating at +-448 (reading R5); the sign bit is kept, so -0 and negative
 * values that round to zero give 0x80.  The positive finite codes 0x00..0x7E
 * are ordered by value, so the two neighbours come from a binary search. */
uint8_t orc_e4m3_encode(float y) {
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    double a = fabs((double)y);
    if (a >= 448.0) return sign | 0x7E;
    int lo = 0, hi = 0x7E; /* value(lo) <= a < value(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (orc_e4m3_value((uint8_t)mid) <= a) lo = mid; else hi = mid;
    }
    double dlo = a - orc_e4m3_value((uint8_t)lo);
    double dhi = orc_e4m3_value((uint8_t)hi) - a;
    int c;
    if (dlo < dhi) c = lo;
    else if (dhi < dlo) c = hi;
    else c = (lo & 1) ? hi : lo;
    return sign | (uint8_t)c;
}

/* [P1] e2m1_index: |v| clamped to 6, then the nearest grid magnitude, a tie
 * going to the even code index.  Written as the definition: argmin over the
 * grid (distances are exact in fp64). */
int orc_e2m1_index(float a_in) {
    float a = a_in < 6.0f ? a_in : 6.0f;
    int best = 0;
    double bd = fabs((double)a - (double)E2M1_GRID[0]);
    for (int i = 1; i < 8; ++i) {
        double d = fabs((double)a - (double)E2M1_GRID[i]);
        if (d < bd || (d == bd && (i % 2) == 0)) {
            best = i;
            bd = d;
        }
    }
    return best;
}

/* [P1] _block_exponent, reading R1.  amax is clamped below at the smallest
 * normal fp32 as the page does; amax == 0 gives 0; the result is clamped to
 * [-127, 127].
 *   ocp:    floor(log2 amax) - 2        (amax / 2^e lands in [4, 8))
 *   noclip: least e with amax <= 6*2^e  (amax / 2^e lands in (3, 6]) */
int orc_block_exponent(float amax, int mode) {
    if (!(amax > 0.0f)) return 0;
    float safe = amax < FLT_MIN ? FLT_MIN : amax;
    int x;
    frexpf(safe, &x);           /* safe = f * 2^x, f in [0.5, 1) */
    int p = x - 1;              /* floor(log2 safe), exact */
    int e;
    if (mode == ORC_OCP) {
        e = p - 2;
    } else {
        e = p - 3;              /* 6 * 2^(p-3) < 2^p <= safe: never enough */
        while ((double)safe > ldexp(6.0, e)) ++e;
    }
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* [P1] _encode_blocks for one 32-block at exponent e:
 *   v = w / 2^e, idx = e2m1_index(|v|), q = grid[idx] * sign(v) * 2^e,
 *   err = sum (q - w)^2   (summation order: reading R2). */
float orc_encode_block(const float *w, int e, uint8_t *idx) {
    float scale = ldexpf(1.0f, e);      /* 2^e; 2^-127 and 2^-128 are exact subnormals */
    float err = 0.0f;
    for (int j = 0; j < 32; ++j) {
        float v = w[j] / scale;
        int i = orc_e2m1_index(fabsf(v));
        float sgn = (v > 0.0f) ? 1.0f : ((v < 0.0f) ? -1.0f : 0.0f);
        float q = E2M1_GRID[i] * sgn * scale;
        float d = q - w[j];
        float sq = d * d;
        err = err + sq;
        idx[j] = (uint8_t)i;
    }
    return err;
}

/* [P1] quant_mxfp4 for one block: block exponent by rule, mse trial of the
 * no-clip exponent and one binade finer (reading R3), then the sign bit only
 * where the index is nonzero (negative zero keeps code 0).  Returns e. */
int orc_quant_block(const float *w, int mode, uint8_t *code, float *err_out) {
    float amax = 0.0f;
    for (int j = 0; j < 32; ++j) {
        float a = fabsf(w[j]);
        if (a > amax) amax = a;
    }
    uint8_t idx[32];
    int e;
    float err;
    if (mode == ORC_MSE) {
        uint8_t idx1[32];
        int e0 = orc_block_exponent(amax, ORC_NOCLIP);
        float r0 = orc_encode_block(w, e0, idx);
        e = e0;
        err = r0;
        if (e0 - 1 >= -127) {
            float r1 = orc_encode_block(w, e0 - 1, idx1);
            if (r1 < r0) {
                e = e0 - 1;
                err = r1;
                memcpy(idx, idx1, 32);
            }
        }
    } else {
        e = orc_block_exponent(amax, mode);
        err = orc_encode_block(w, e, idx);
    }
    for (int j = 0; j < 32; ++j)
        code[j] = idx[j] | ((signbit(w[j]) && idx[j] != 0) ? 8 : 0);
    *err_out = err;
    return e;
}

/* [P1] quant_mxfp4 over rows: [rows, K] fp32 -> packed [rows, K/2] (low
 * nibble = even k), e8m0 [rows, K/32] = e + 127.  block_err (nullable) gets
 * each block's chosen error; err_sum / ssq (nullable) get the sums of block
 * errors and of w^2 in fp64. */
void orc_quant_mxfp4(const float *w, int64_t rows, int64_t K, int mode,
                     uint8_t *packed, uint8_t *e8m0, float *block_err,
                     double *err_sum, double *ssq) {
    int64_t nb = K / 32;
    double *row_err = (double *)calloc((size_t)(rows > 0 ? rows : 1), sizeof(double));
    double *row_ssq = (double *)calloc((size_t)(rows > 0 ? rows : 1), sizeof(double));
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double re = 0.0, rs = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            const float *wb = w + r * K + b * 32;
            uint8_t code[32];
            float err;
            int e = orc_quant_block(wb, mode, code, &err);
            for (int j = 0; j < 16; ++j)
                packed[r * (K / 2) + b * 16 + j] = (uint8_t)(code[2 * j] | (code[2 * j + 1] << 4));
            e8m0[r * nb + b] = (uint8_t)(e + 127);
            if (block_err) block_err[r * nb + b] = err;
            re += (double)err;
            for (int j = 0; j < 32; ++j) rs += (double)wb[j] * (double)wb[j];
        }
        row_err[r] = re;
        row_ssq[r] = rs;
    }
    double te = 0.0, ts = 0.0;
    for (int64_t r = 0; r < rows; ++r) {
        te += row_err[r];
        ts += row_ssq[r];
    }
    if (err_sum) *err_sum = te;
    if (ssq) *ssq = ts;
    free(row_err);
    free(row_ssq);
}

/* [P1] dequant_mxfp4: w = e2m1 * 2^(byte - 127), exact in fp32 (2^-127 is
 * a subnormal power of two). */
void orc_dequant_mxfp4(const uint8_t *packed, const uint8_t *e8m0,
                       int64_t rows, int64_t K, float *w) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k) {
            uint8_t byte = packed[r * (K / 2) + k / 2];
            int code = (k & 1) ? (byte >> 4) : (byte & 15);
            float scale = ldexpf(1.0f, (int)e8m0[r * (K / 32) + k / 32] - 127);
            w[r * K + k] = orc_e2m1_value(code) * scale;
        }
}

/* ------------------------------------------------------------------------ */
/* NVFP4 -> MXFP4                                                            */
/* ------------------------------------------------------------------------ */

/* [P1] dequant_nvfp4: W[n,k] = e2m1 * (fp32(scale[n, k/16]) / divisor), the
 * divisor being the checkpoint's global scale as stored (6*448/amax).
 * Reading R4: divide first (IEEE fp32), then multiply. */
void orc_dequant_nvfp4(const uint8_t *packed, const uint8_t *scale,
                       int64_t rows, int64_t K, float divisor, float *w) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k) {
            uint8_t byte = packed[r * (K / 2) + k / 2];
            int code = (k & 1) ? (byte >> 4) : (byte & 15);
            float s = (float)orc_e4m3_value(scale[r * (K / 16) + k / 16]) / divisor;
            w[r * K + k] = orc_e2m1_value(code) * s;
        }
}

/* [P1] RadianceNvfp4ToMxfp4.process_weights_after_loading with requant_rows:
 * each partition (a consecutive row range with its own divisor) is
 * dequantized and re-encoded in passes of row_chunk rows (0 = whole
 * partition); outputs are concatenated in row order.  stats (nullable):
 * per partition {sum of chosen block errors, sum of w^2}, fp64.
 * Returns 0, or -1 on a bad argument (K % 32, row sums, divisors). */
int orc_requant_nvfp4_to_mxfp4(const uint8_t *nv_packed, const uint8_t *nv_scale,
                               const int64_t *part_rows, const float *part_divisor,
                               int n_parts, int64_t K, int mode, int64_t row_chunk,
                               uint8_t *mx_packed, uint8_t *mx_e8m0, double *stats) {
    if (K <= 0 || K % 32 != 0 || n_parts < 1) return -1;
    int64_t r0 = 0;
    for (int p = 0; p < n_parts; ++p) {
        int64_t width = part_rows[p];
        float gd = part_divisor[p];
        if (width < 0 || !(gd > 0.0f) || !isfinite(gd)) return -1;
        int64_t chunk = row_chunk > 0 ? row_chunk : (width > 0 ? width : 1);
        double err = 0.0, ssq = 0.0;
        for (int64_t a = 0; a < width; a += chunk) {
            int64_t n = (width - a) < chunk ? (width - a) : chunk;
            int64_t r = r0 + a;
            float *w = (float *)malloc((size_t)(n * K) * sizeof(float));
            if (!w) return -1;
            orc_dequant_nvfp4(nv_packed + r * (K / 2), nv_scale + r * (K / 16), n, K, gd, w);
            double e = 0.0, s = 0.0;
            orc_quant_mxfp4(w, n, K, mode, mx_packed + r * (K / 2), mx_e8m0 + r * (K / 32),
                            NULL, &e, &s);
            err += e;
            ssq += s;
            free(w);
        }
        if (stats) {
            stats[2 * p] = err;
            stats[2 * p + 1] = ssq;
        }
        r0 += width;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* bf16 and fp8 per-channel weights -> MXFP4                                 */
/* ------------------------------------------------------------------------ */

/* [P1] RadianceBf16ToMxfp4.process_weights_after_loading: requant_rows on the
 * bf16 weight itself -- each element widened to fp32 (exact), then
 * quant_mxfp4 over rows.  The ROW_CHUNK passes do not change any output.
 * stats (nullable): {sum of chosen block errors, sum of w^2}, fp64.
 * Returns 0, or -1 on a bad argument (K % 32) or a non-finite input. */
int orc_quant_bf16_to_mxfp4(const uint16_t *w_bf16, int64_t rows, int64_t K, int mode,
                            uint8_t *mx_packed, uint8_t *mx_e8m0, double *stats) {
    if (rows < 0 || K <= 0 || K % 32 != 0) return -1;
    float *w = (float *)malloc((size_t)((rows > 0 ? rows : 1) * K) * sizeof(float));
    if (!w) return -1;
    int bad = 0;
    for (int64_t i = 0; i < rows * K; ++i) {
        w[i] = orc_bf16_value(w_bf16[i]);
        if (!isfinite(w[i])) bad = 1;
    }
    if (!bad) {
        double e = 0.0, s = 0.0;
        orc_quant_mxfp4(w, rows, K, mode, mx_packed, mx_e8m0, NULL, &e, &s);
        if (stats) {
            stats[0] = e;
            stats[1] = s;
        }
    }
    free(w);
    return bad ? -1 : 0;
}

/* [P1] RadianceFp8ChannelToMxfp4.process_weights_after_loading: the e4m3
 * weight widened to fp32 and multiplied by its row's fp32 scale (one
 * correctly rounded fp32 product), then quant_mxfp4 over rows.  stats as
 * above.  Returns 0, or -1 on a bad argument or a NaN code / non-finite
 * scale. */
int orc_quant_fp8ch_to_mxfp4(const uint8_t *w_e4m3, const float *row_scale, int64_t rows,
                             int64_t K, int mode, uint8_t *mx_packed, uint8_t *mx_e8m0,
                             double *stats) {
    if (rows < 0 || K <= 0 || K % 32 != 0) return -1;
    float *w = (float *)malloc((size_t)((rows > 0 ? rows : 1) * K) * sizeof(float));
    if (!w) return -1;
    int bad = 0;
    for (int64_t r = 0; r < rows; ++r) {
        const float s = row_scale[r];
        if (!isfinite(s)) bad = 1;
        for (int64_t k = 0; k < K; ++k) {
            const double v = orc_e4m3_value(w_e4m3[r * K + k]);
            if (!isfinite(v)) bad = 1;
            w[r * K + k] = (float)v * s;
        }
    }
    if (!bad) {
        double e = 0.0, ss = 0.0;
        orc_quant_mxfp4(w, rows, K, mode, mx_packed, mx_e8m0, NULL, &e, &ss);
        if (stats) {
            stats[0] = e;
            stats[1] = ss;
        }
    }
    free(w);
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* per-token fp8 activations (reading R5)                                    */
/* ------------------------------------------------------------------------ */

/* [P3] autoround_linear: activations become e4m3 codes with one fp32 scale
 * per token (row).  Returns 0, or -1 if an input is not finite. */
int orc_quant_act_fp8(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                      uint8_t *x8, float *x_scale) {
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t m = 0; m < M; ++m) {
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float v = orc_bf16_value(x[m * ldx + k]);
            if (!isfinite(v)) bad = 1;
            float a = fabsf(v);
            if (a > amax) amax = a;
        }
        float s = (amax > 0.0f) ? amax / 448.0f : 1.0f;
        x_scale[m] = s;
        for (int64_t k = 0; k < K; ++k) {
            float y = orc_bf16_value(x[m * ldx + k]) / s;
            x8[m * K + k] = orc_e4m3_encode(y);
        }
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* GEMM references (reading R6)                                              */
/* ------------------------------------------------------------------------ */

/* [P3] _exact_ref, with the MXFP4 dequant of [P1] dequant_mxfp4:
 *   ref[m,n] = s_m * sum_k dec(x8[m,k]) * e2m1(w[n,k]) * 2^(E[n,k/32]-127).
 * With mi == NULL the full [M,N] is written row-major; otherwise ref[i] is
 * the output at (mi[i], ni[i]) for i < count. */
static double mx_dot(const uint8_t *x8, const uint8_t *wp, const uint8_t *we,
                     int64_t m, int64_t n, int64_t K) {
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        uint8_t byte = wp[n * (K / 2) + k / 2];
        int code = (k & 1) ? (byte >> 4) : (byte & 15);
        double wv = (double)orc_e2m1_value(code) * ldexp(1.0, (int)we[n * (K / 32) + k / 32] - 127);
        acc += orc_e4m3_value(x8[m * K + k]) * wv;
    }
    return acc;
}

void orc_mxfp4_gemm(const uint8_t *x8, const float *x_scale, const uint8_t *w_packed,
                    const uint8_t *w_e8m0, int64_t M, int64_t N, int64_t K,
                    const int64_t *mi, const int64_t *ni, int64_t count, double *ref) {
    if (!mi) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t m = 0; m < M; ++m)
                ref[m * N + n] = (double)x_scale[m] * mx_dot(x8, w_packed, w_e8m0, m, n, K);
    } else {
#pragma omp parallel for schedule(dynamic, 16)
        for (int64_t i = 0; i < count; ++i)
            ref[i] = (double)x_scale[mi[i]] * mx_dot(x8, w_packed, w_e8m0, mi[i], ni[i], K);
    }
}

/* [P2] MXFP4 checkpoints with MXFP4 activations (the declared W4A4 numerics
 * the page's W4A8 kernel departs from): activations quantized per token and
 * 32-block to e2m1 + e8m0, weights e2m1 + e8m0;
 *   out[m,n] = sum_k e2m1(x[m,k]) 2^(Ex[m,k/32]-127) * e2m1(w[n,k]) 2^(Ew[n,k/32]-127),
 * exact products, fp64 accumulation, not rounded. */
static double w4a4_dot(const uint8_t *xp, const uint8_t *xe, const uint8_t *wp, const uint8_t *we,
                       int64_t m, int64_t n, int64_t K) {
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        uint8_t xb = xp[m * (K / 2) + k / 2], wb = wp[n * (K / 2) + k / 2];
        int xc = (k & 1) ? (xb >> 4) : (xb & 15), wc = (k & 1) ? (wb >> 4) : (wb & 15);
        double xv = (double)orc_e2m1_value(xc) * ldexp(1.0, (int)xe[m * (K / 32) + k / 32] - 127);
        double wv = (double)orc_e2m1_value(wc) * ldexp(1.0, (int)we[n * (K / 32) + k / 32] - 127);
        acc += xv * wv;
    }
    return acc;
}

void orc_w4a4_gemm(const uint8_t *x_packed, const uint8_t *x_e8m0, const uint8_t *w_packed,
                   const uint8_t *w_e8m0, int64_t M, int64_t N, int64_t K,
                   const int64_t *mi, const int64_t *ni, int64_t count, double *ref) {
    if (!mi) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t m = 0; m < M; ++m)
                ref[m * N + n] = w4a4_dot(x_packed, x_e8m0, w_packed, w_e8m0, m, n, K);
    } else {
#pragma omp parallel for schedule(dynamic, 16)
        for (int64_t i = 0; i < count; ++i)
            ref[i] = w4a4_dot(x_packed, x_e8m0, w_packed, w_e8m0, mi[i], ni[i], K);
    }
}

/* [P3] process_weights_after_loading: every qzeros word must be 0x77777777
 * (zero point 8, symmetric); the weight is transposed from [K/8, N] to
 * [N, K/8].  Returns the number of qzeros words that differ (0 = accepted);
 * the transpose is written only when that number is 0. */
int orc_int4_prepare(const int32_t *qweight_kn, const int32_t *qzeros,
                     int64_t N, int64_t K, int32_t *qweight_nk) {
    int64_t nz = (K / 128) * (N / 8);
    int64_t bad = 0;
    for (int64_t i = 0; i < nz; ++i)
        if ((uint32_t)qzeros[i] != 0x77777777u) ++bad;
    if (bad) return bad > 0x7fffffff ? 0x7fffffff : (int)bad;
    for (int64_t i = 0; i < K / 8; ++i)
        for (int64_t n = 0; n < N; ++n)
            qweight_nk[n * (K / 8) + i] = qweight_kn[i * N + n];
    return 0;
}

/* [P3] _exact_ref: code c = nibble (k % 8) of word [n, k/8]; weight
 * (c - 8) * fp32(scales[k/128, n]); then as the MXFP4 reference. */
static double i4_dot(const uint8_t *x8, const int32_t *qw, const uint16_t *sc,
                     int64_t m, int64_t n, int64_t N, int64_t K) {
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        uint32_t word = (uint32_t)qw[n * (K / 8) + k / 8];
        int c = (int)((word >> (4 * (k % 8))) & 15u);
        double wv = (double)(c - 8) * orc_f16_value(sc[(k / 128) * N + n]);
        acc += orc_e4m3_value(x8[m * K + k]) * wv;
    }
    return acc;
}

void orc_int4_gemm(const uint8_t *x8, const float *x_scale, const int32_t *qweight_nk,
                   const uint16_t *scales_f16, int64_t M, int64_t N, int64_t K,
                   const int64_t *mi, const int64_t *ni, int64_t count, double *ref) {
    if (!mi) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t m = 0; m < M; ++m)
                ref[m * N + n] = (double)x_scale[m] * i4_dot(x8, qweight_nk, scales_f16, m, n, N, K);
    } else {
#pragma omp parallel for schedule(dynamic, 16)
        for (int64_t i = 0; i < count; ++i)
            ref[i] = (double)x_scale[mi[i]] * i4_dot(x8, qweight_nk, scales_f16, mi[i], ni[i], N, K);
    }
}

/* int4 g128 with a zero point per group and column (asymmetric): "vllm-radiance
 * (MXFP4)", ParoQuant (int4 W4A8 and int5 W5A8): int4 group-128 asymmetric
 * weights on the W4A8 path; the checkpoint layout and zero convention of
 * "radiance_autoround.py", module docstring: qweight [K/8, N] with eight
 * codes along K (nibble k % 8 of word [k/8, n]), scales [K/128, N] fp16,
 * qzeros [K/128, N/8] with eight zero points along N, each stored minus one
 * (nibble n % 8 of word [k/128, n/8] is z - 1).  Weight (c - z) * scale;
 * then as the MXFP4 reference. */
static double i4zp_dot(const uint8_t *x8, const int32_t *qw_kn, const int32_t *qz, const uint16_t *sc,
                       int64_t m, int64_t n, int64_t N, int64_t K) {
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        uint32_t word = (uint32_t)qw_kn[(k / 8) * N + n];
        int c = (int)((word >> (4 * (k % 8))) & 15u);
        uint32_t zw = (uint32_t)qz[(k / 128) * (N / 8) + n / 8];
        int z = (int)((zw >> (4 * (n % 8))) & 15u) + 1;
        double wv = (double)(c - z) * orc_f16_value(sc[(k / 128) * N + n]);
        acc += orc_e4m3_value(x8[m * K + k]) * wv;
    }
    return acc;
}

void orc_int4_zp_gemm(const uint8_t *x8, const float *x_scale, const int32_t *qweight_kn,
                      const int32_t *qzeros, const uint16_t *scales_f16, int64_t M, int64_t N, int64_t K,
                      const int64_t *mi, const int64_t *ni, int64_t count, double *ref) {
    if (!mi) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t m = 0; m < M; ++m)
                ref[m * N + n] = (double)x_scale[m] * i4zp_dot(x8, qweight_kn, qzeros, scales_f16, m, n, N, K);
    } else {
#pragma omp parallel for schedule(dynamic, 16)
        for (int64_t i = 0; i < count; ++i)
            ref[i] = (double)x_scale[mi[i]] * i4zp_dot(x8, qweight_kn, qzeros, scales_f16, mi[i], ni[i], N, K);
    }
}

/* int5 g128 (W5A8): "vllm-radiance (MXFP4)", int5 (W5A8): 5-bit ParoQuant
 * codes on the W4A8 path, the zero point folded as for int4.  The pages
 * describe the kernel's staging (low nibbles in the int4 word layout, the
 * fifth bit in a plane of its own) but print no checkpoint layout; the
 * reading here: qweight [K/8, N] holds the low four bits of each code as the
 * int4 layout, qweight_hi [K/32, N] the fifth bits (bit k % 32 of word
 * [k/32, n] is bit 4 of code k), qzeros [K/128, N] one byte per group and
 * column holding z - 1 (the zero stored minus one, as the int4 checkpoints),
 * scales [K/128, N] fp16.  Weight (c - z) * scale, c = low | fifth << 4. */
static double i5_dot(const uint8_t *x8, const int32_t *qw_kn, const int32_t *qh_kn, const uint8_t *qz,
                     const uint16_t *sc, int64_t m, int64_t n, int64_t N, int64_t K) {
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        uint32_t lo = ((uint32_t)qw_kn[(k / 8) * N + n] >> (4 * (k % 8))) & 15u;
        uint32_t hi = ((uint32_t)qh_kn[(k / 32) * N + n] >> (k % 32)) & 1u;
        int c = (int)(lo | (hi << 4));
        int z = (int)qz[(k / 128) * N + n] + 1;
        double wv = (double)(c - z) * orc_f16_value(sc[(k / 128) * N + n]);
        acc += orc_e4m3_value(x8[m * K + k]) * wv;
    }
    return acc;
}

void orc_int5_gemm(const uint8_t *x8, const float *x_scale, const int32_t *qweight_kn, const int32_t *qweight_hi,
                   const uint8_t *qzeros, const uint16_t *scales_f16, int64_t M, int64_t N, int64_t K,
                   const int64_t *mi, const int64_t *ni, int64_t count, double *ref) {
    if (!mi) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t m = 0; m < M; ++m)
                ref[m * N + n] = (double)x_scale[m] *
                                 i5_dot(x8, qweight_kn, qweight_hi, qzeros, scales_f16, m, n, N, K);
    } else {
#pragma omp parallel for schedule(dynamic, 16)
        for (int64_t i = 0; i < count; ++i)
            ref[i] = (double)x_scale[mi[i]] *
                     i5_dot(x8, qweight_kn, qweight_hi, qzeros, scales_f16, mi[i], ni[i], N, K);
    }
}

/* ------------------------------------------------------------------------ */
/* array forms of the scalar functions above (loops only, for sweeps)        */
/* ------------------------------------------------------------------------ */

void orc_e2m1_index_array(const float *a, int64_t n, uint8_t *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_e2m1_index(a[i]);
}

void orc_block_exponent_array(const float *amax, int64_t n, int mode, int32_t *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_block_exponent(amax[i], mode);
}

void orc_e4m3_encode_array(const float *y, int64_t n, uint8_t *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(y[i]);
}
