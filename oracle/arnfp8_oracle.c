/*
 * arnfp8_oracle.c -- plain, slow, single-threaded CPU oracle for the fused
 * all-reduce sum + residual + RMSNorm + per-row dynamic FP8 quantisation
 * epilogue.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this code.  It shares nothing
 * with the GPU path.  Build: gcc -O2 -std=c11 -ffp-contract=off (no fast-math:
 * every fp32 operation below must be one IEEE-754 rounding in the order shown).
 *
 * What the operation computes, and where it comes from:
 *  - Sum of the per-GPU input buffers, then RMSNorm with gamma and an additive
 *    weight offset and epsilon, then FP8 dynamic quantisation with one fp32
 *    scale per row (last dim 1), the scale bounded above by scale_ub:
 *    Modular Mojo API docs, "allreduce_rmsnorm_fp8" (function summary; Args:
 *    input_buffers, output, gamma, epsilon, weight_offset, scale_ub,
 *    scale_output).
 *  - The sum is accumulated in fp32 in a fixed rank order and rounded to bf16
 *    once: b12x PR #283 "PCIeTwoShotBF16" (PR description; Validation,
 *    "Precision").
 *  - A residual is added before the norm and the updated residual is written
 *    back (the RESIDUAL_RMS_NORM epilogue): TensorRT-LLM PR #19836
 *    (Description).
 *  - weight_offset = 1 gives the unit-offset gain 1 + gamma: tt-metal
 *    rmsnorm_2d.py (RMSNorm2DConfig.add_unit_offset, "e.g., for Gemma").
 *  - Per-row ("per-token") dynamic quantisation to E4M3FN / E5M2: Huawei CANN
 *    aclnnAlltoAllQuantMatmul (x1QuantMode, x1QuantDtype).
 *
 * Readings where the pages are silent (each one is listed in the design
 * notes): the residual adds the *rounded* bf16 sum; the norm reads the rounded
 * bf16 h; the fp32 accumulator starts from rank 0's value (so -0 survives
 * P = 1); gamma + weight_offset is one fp32 add (not re-rounded to bf16); eps
 * is added to the mean square inside the square root; amax is taken over the
 * post-gain normalised row; the fp8 code is decided from an fp32 value
 * (fl32(y / scale)), round-to-nearest-even with saturation at +-448; with
 * eps = 0 an all-zero row normalises to y = 0 (floor scale, zero codes); eps
 * must be finite and >= 0, weight_offset finite and scale_ub > 0 (calls with
 * other values return ORACLE_BAD_ARG).
 *
 * The norm statistics and the normalised row are computed in fp64, so the
 * oracle's y is the exact value up to a few fp64 roundings.
 */
#include "arnfp8_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- bf16 -- */

float oracle_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16; /* bf16 is the top half of an fp32 */
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if (isnan(f))
        return (uint16_t)((u >> 16) | 0x0040u); /* keep sign, force quiet */

    /* The kept half truncates toward zero; the dropped half decides.  More
     * than half an ulp -> away from zero; exactly half -> to the even kept
     * half.  A carry out of the mantissa correctly bumps the exponent (and
     * the largest finite values overflow to inf, as rounding demands). */
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xFFFFu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))
        kept += 1u;
    return (uint16_t)kept;
}

/* ------------------------------------------------------ small floats -- */
/*
 * A sign-magnitude binary float with E exponent bits, M mantissa bits and
 * exponent bias B.  e4m3fn: E=4, M=3, B=7, top code 0x7F is NaN, no inf, max
 * finite 1.75 * 2^8 = 448.  e5m2: E=5, M=2, B=15, IEEE-like (inf and NaN in
 * the top exponent), max finite 1.75 * 2^15 = 57344.
 */

/* Round a non-negative finite magnitude to the nearest multiple of the
 * format's spacing at that magnitude, ties to the even multiple.  `emin` is
 * the exponent of the smallest normal number and `mbits` the mantissa width;
 * below 2^emin the spacing stays 2^(emin - mbits) (subnormals). */
static double round_to_grid(double a, int emin, int mbits)
{
    int e;
    if (a < ldexp(1.0, emin)) {
        e = emin;
    } else {
        int k;
        (void)frexp(a, &k); /* a = m * 2^k, m in [0.5, 1) */
        e = k - 1;          /* a in [2^e, 2^(e+1)) */
    }
    double quantum = ldexp(1.0, e - mbits);
    double n = a / quantum; /* exact: division by a power of two */
    double lo = floor(n);
    double frac = n - lo;
    if (frac > 0.5 || (frac == 0.5 && fmod(lo, 2.0) == 1.0))
        lo += 1.0;
    return lo * quantum; /* may be 2^(e+1): the next binade, still exact */
}

/* Bit pattern of a non-negative value that is exactly representable. */
static uint8_t encode_exact(double v, int emin, int mbits, int bias)
{
    if (v == 0.0)
        return 0;
    if (v < ldexp(1.0, emin)) { /* subnormal: exponent field 0 */
        double m = v / ldexp(1.0, emin - mbits);
        return (uint8_t)m;
    }
    int k;
    double m = frexp(v, &k);    /* v = m * 2^k, m in [0.5, 1) */
    int e = k - 1;              /* v = (2m) * 2^e, 2m in [1, 2) */
    double frac = (2.0 * m - 1.0) * ldexp(1.0, mbits);
    return (uint8_t)(((e + bias) << mbits) | (int)frac);
}

static double decode_small(uint8_t code, int ebits, int mbits, int bias)
{
    int sign = (code >> (ebits + mbits)) & 1;
    int efield = (code >> mbits) & ((1 << ebits) - 1);
    int mfield = code & ((1 << mbits) - 1);
    double v;
    if (efield == 0)
        v = ldexp((double)mfield, 1 - bias - mbits);
    else
        v = ldexp(1.0 + ldexp((double)mfield, -mbits), efield - bias);
    return sign ? -v : v;
}

double oracle_e4m3fn_to_f64(uint8_t code)
{
    if ((code & 0x7F) == 0x7F)
        return NAN; /* S.1111.111 is the only NaN; there is no inf */
    return decode_small(code, 4, 3, 7);
}

uint8_t oracle_f32_to_e4m3fn_sat(float v)
{
    if (isnan(v))
        return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a >= 448.0)
        return sign | 0x7E; /* saturate at the largest finite value */
    double r = round_to_grid(a, -6, 3); /* a < 448 rounds to at most 448 */
    return sign | encode_exact(r, -6, 3, 7);
}

double oracle_e5m2_to_f64(uint8_t code)
{
    int efield = (code >> 2) & 0x1F;
    if (efield == 0x1F) {
        if (code & 0x3)
            return NAN;
        return (code & 0x80) ? -INFINITY : INFINITY;
    }
    return decode_small(code, 5, 2, 15);
}

uint8_t oracle_f32_to_e5m2_sat(float v)
{
    if (isnan(v))
        return 0x7E;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a >= 57344.0)
        return sign | 0x7B; /* saturate at the largest finite value */
    double r = round_to_grid(a, -14, 2); /* a < 57344 rounds to <= 57344 */
    return sign | encode_exact(r, -14, 2, 15);
}

/* ------------------------------------------------------ the operation -- */

static int check_common(const uint16_t *const *inputs, int P, int64_t rows,
                        int64_t cols)
{
    if (inputs == NULL || P < 1 || P > 8 || rows < 0 || cols <= 0)
        return ORACLE_BAD_ARG;
    for (int p = 0; p < P; ++p)
        if (inputs[p] == NULL)
            return ORACLE_BAD_ARG;
    return ORACLE_OK;
}

/* The norm's scalars: epsilon is a stabilising term added to the mean square,
 * so it must be finite and not negative; the weight offset is added to gamma,
 * so it must be finite; scale_ub bounds the scale from above, so it must be
 * positive (+inf: no bound).  `check_ub` is 0 for the MX output, which has no
 * scale_ub. */
static int check_scalars(float eps, float weight_offset, float scale_ub, int check_ub)
{
    if (!isfinite(eps) || eps < 0.0f || !isfinite(weight_offset))
        return ORACLE_BAD_ARG;
    if (check_ub && !(scale_ub > 0.0f))
        return ORACLE_BAD_ARG;
    return ORACLE_OK;
}

/* One element of the rank-order sum: start from rank 0's value, add ranks
 * 1..P-1 in order, each add one fp32 rounding; round the total to bf16 once. */
static uint16_t rank_order_sum(const uint16_t *const *inputs, int P, int64_t k)
{
    float acc = oracle_bf16_to_f32(inputs[0][k]);
    for (int p = 1; p < P; ++p)
        acc = acc + oracle_bf16_to_f32(inputs[p][k]);
    return oracle_f32_to_bf16(acc);
}

int oracle_sum_bf16(const uint16_t *const *inputs, int P, uint16_t *out,
                    int64_t rows, int64_t cols)
{
    int st = check_common(inputs, P, rows, cols);
    if (st != ORACLE_OK || out == NULL)
        return st != ORACLE_OK ? st : ORACLE_BAD_ARG;
    for (int64_t k = 0; k < rows * cols; ++k)
        out[k] = rank_order_sum(inputs, P, k);
    return ORACLE_OK;
}

/* Steps S1-S5 for row i: sum, optional residual add and write-back, and the
 * normalised row y = h * r * g in fp64.  `h` and `y` hold `cols` doubles. */
static void norm_row(const uint16_t *const *inputs, int P, const uint16_t *residual_in,
                     uint16_t *residual_out, const uint16_t *gamma, float eps,
                     float weight_offset, int64_t i, int64_t cols, double *h, double *y)
{
    /* Sum, optional residual add, residual write-back. */
    for (int64_t j = 0; j < cols; ++j) {
        int64_t k = i * cols + j;
        uint16_t hb = rank_order_sum(inputs, P, k);
        if (residual_in != NULL) {
            float t = oracle_bf16_to_f32(hb) + oracle_bf16_to_f32(residual_in[k]);
            hb = oracle_f32_to_bf16(t);
        }
        if (residual_out != NULL)
            residual_out[k] = hb;
        h[j] = (double)oracle_bf16_to_f32(hb);
    }

    /* RMSNorm: r = 1 / sqrt(mean(h^2) + eps), y = h * r * g.  With eps = 0
     * an all-zero row has mean(h^2) + eps = 0 and nothing to normalise: the
     * reading taken is y = 0 (so the row gets the floor scale and zero codes,
     * never a NaN).  In fp64 the sum of squares of bf16 values is zero only
     * when every h is zero, so no other row takes this branch. */
    double sumsq = 0.0;
    for (int64_t j = 0; j < cols; ++j)
        sumsq += h[j] * h[j];
    double ms = sumsq / (double)cols;
    double den = ms + (double)eps;
    double r = den > 0.0 ? 1.0 / sqrt(den) : 0.0;

    for (int64_t j = 0; j < cols; ++j) {
        float g = oracle_bf16_to_f32(gamma[j]) + weight_offset; /* fp32 add */
        y[j] = h[j] * r * (double)g;
    }
}

/* Per-row scale: amax clamped at scale_ub, over the format's maximum `fmax`,
 * floored at 1 / (fmax * 512); all in fp32 (fmax * 512 is exact). */
static float row_scale(float amax, float scale_ub, float fmax)
{
    return fmaxf(fminf(amax, scale_ub) / fmax, 1.0f / (fmax * 512.0f));
}

/* The per-row dynamic quantisation shared by the e4m3fn and e5m2 outputs. */
static int fused_per_row(const uint16_t *const *inputs, int P, const uint16_t *residual_in,
                         uint16_t *residual_out, uint8_t *out_fp8, float *scales,
                         const uint16_t *gamma, float eps, float weight_offset,
                         float scale_ub, int64_t rows, int64_t cols, int e5m2)
{
    int st = check_common(inputs, P, rows, cols);
    if (st != ORACLE_OK)
        return st;
    if (out_fp8 == NULL || scales == NULL || gamma == NULL)
        return ORACLE_BAD_ARG;

    if (check_scalars(eps, weight_offset, scale_ub, 1) != ORACLE_OK)
        return ORACLE_BAD_ARG;

    const float fmax = e5m2 ? 57344.0f : 448.0f;
    double *h = (double *)malloc((size_t)cols * sizeof(double));
    double *y = (double *)malloc((size_t)cols * sizeof(double));
    if (h == NULL || y == NULL) {
        free(h);
        free(y);
        return ORACLE_NO_MEMORY;
    }

    for (int64_t i = 0; i < rows; ++i) {
        norm_row(inputs, P, residual_in, residual_out, gamma, eps, weight_offset, i, cols, h, y);

        double ymax = 0.0;
        for (int64_t j = 0; j < cols; ++j)
            if (fabs(y[j]) > ymax)
                ymax = fabs(y[j]);
        float amax = (float)ymax;
        float scale = row_scale(amax, scale_ub, fmax);
        scales[i] = scale;

        /* Quantise: the code is decided from the fp32 value y / scale. */
        for (int64_t j = 0; j < cols; ++j) {
            float v = (float)(y[j] / (double)scale);
            if (v > fmax)
                v = fmax;
            if (v < -fmax)
                v = -fmax;
            out_fp8[i * cols + j] = e5m2 ? oracle_f32_to_e5m2_sat(v) : oracle_f32_to_e4m3fn_sat(v);
        }
    }

    free(h);
    free(y);
    return ORACLE_OK;
}

int oracle_arnfp8(const uint16_t *const *inputs, int P,
                  const uint16_t *residual_in, uint16_t *residual_out,
                  uint8_t *out_fp8, float *scales, const uint16_t *gamma,
                  float eps, float weight_offset, float scale_ub,
                  int64_t rows, int64_t cols)
{
    return fused_per_row(inputs, P, residual_in, residual_out, out_fp8, scales, gamma, eps,
                         weight_offset, scale_ub, rows, cols, 0);
}

int oracle_arnfp8_e5m2(const uint16_t *const *inputs, int P,
                       const uint16_t *residual_in, uint16_t *residual_out,
                       uint8_t *out_fp8, float *scales, const uint16_t *gamma,
                       float eps, float weight_offset, float scale_ub,
                       int64_t rows, int64_t cols)
{
    return fused_per_row(inputs, P, residual_in, residual_out, out_fp8, scales, gamma, eps,
                         weight_offset, scale_ub, rows, cols, 1);
}

int oracle_norm_rows(const uint16_t *const *inputs, int P, const uint16_t *residual_in,
                     uint16_t *residual_out, const uint16_t *gamma, float eps,
                     float weight_offset, int64_t rows, int64_t cols, double *y)
{
    int st = check_common(inputs, P, rows, cols);
    if (st != ORACLE_OK)
        return st;
    if (gamma == NULL || y == NULL || check_scalars(eps, weight_offset, 0.0f, 0) != ORACLE_OK)
        return ORACLE_BAD_ARG;
    double *h = (double *)malloc((size_t)cols * sizeof(double));
    if (h == NULL)
        return ORACLE_NO_MEMORY;
    for (int64_t i = 0; i < rows; ++i)
        norm_row(inputs, P, residual_in, residual_out, gamma, eps, weight_offset, i, cols, h,
                 y + i * cols);
    free(h);
    return ORACLE_OK;
}

/* ------------------------------------------------- MX block quantisation -- */
/*
 * OCP Microscaling (MX) v1.0, MXFP8 with E4M3 elements: a block of 32 values
 * shares one power-of-two scale X = 2^e stored as an E8M0 byte (e + 127).
 * e = floor(log2(max_i |V_i|)) - emax, with emax = 8 the exponent of the
 * largest E4M3 normal (448 = 1.75 * 2^8); each element is V_i / X rounded to
 * E4M3 (nearest, ties to even), saturating at +-448.  A block of zeros takes
 * e = -127 (the smallest E8M0 scale).  The block structure follows the
 * mx-quantisation scale shape (BS, ceil(H/64), 2) of Huawei CANN
 * aclnnAlltoAllQuantMatmul (calculation formula): two scales per 64 values.
 */

int oracle_mx_shared_exp(const double *v, int n)
{
    double amax = 0.0;
    for (int i = 0; i < n; ++i)
        if (fabs(v[i]) > amax)
            amax = fabs(v[i]);
    if (amax == 0.0)
        return -127;
    int k;
    (void)frexp(amax, &k);  /* amax = m * 2^k, m in [0.5, 1): floor(log2) = k - 1 */
    int e = (k - 1) - 8;
    if (e < -127)
        e = -127;
    if (e > 127)
        e = 127;
    return e;
}

void oracle_mx_quantize_block(const double *v, int n, int shared_exp, uint8_t *codes)
{
    for (int i = 0; i < n; ++i) {
        float q = (float)ldexp(v[i], -shared_exp); /* the decision value, in fp32 */
        if (q > 448.0f)
            q = 448.0f;
        if (q < -448.0f)
            q = -448.0f;
        codes[i] = oracle_f32_to_e4m3fn_sat(q);
    }
}

int oracle_arnfp8_mx(const uint16_t *const *inputs, int P,
                     const uint16_t *residual_in, uint16_t *residual_out,
                     uint8_t *out_fp8, uint8_t *block_scales, const uint16_t *gamma,
                     float eps, float weight_offset, int64_t rows, int64_t cols)
{
    int st = check_common(inputs, P, rows, cols);
    if (st != ORACLE_OK)
        return st;
    if (out_fp8 == NULL || block_scales == NULL || gamma == NULL || cols % 32 != 0 ||
        check_scalars(eps, weight_offset, 0.0f, 0) != ORACLE_OK)
        return ORACLE_BAD_ARG;
    double *h = (double *)malloc((size_t)cols * sizeof(double));
    double *y = (double *)malloc((size_t)cols * sizeof(double));
    if (h == NULL || y == NULL) {
        free(h);
        free(y);
        return ORACLE_NO_MEMORY;
    }
    for (int64_t i = 0; i < rows; ++i) {
        norm_row(inputs, P, residual_in, residual_out, gamma, eps, weight_offset, i, cols, h, y);
        for (int64_t b = 0; b < cols / 32; ++b) {
            int e = oracle_mx_shared_exp(y + 32 * b, 32);
            block_scales[i * (cols / 32) + b] = (uint8_t)(e + 127);
            oracle_mx_quantize_block(y + 32 * b, 32, e, out_fp8 + i * cols + 32 * b);
        }
    }
    free(h);
    free(y);
    return ORACLE_OK;
}

/* ------------------------------------------- two-stage share and staging -- */
/*
 * The layout of one rank's slot follows the signal-buffer sizing of the
 * 2-stage path: ceildiv(rows, ngpus) * cols bytes of fp8 data, then the
 * share's scales, ceildiv(rows, ngpus) * sizeof(float) bytes aligned up to
 * the SIMD width (Modular Mojo API docs, "allreduce_rmsnorm_fp8", the note
 * on signal buffer sizing; the signal header itself is not part of the slot).
 */

void oracle_share_rows(int64_t rows, int ngpus, int rank, int64_t *first, int64_t *count)
{
    int64_t S = (rows + ngpus - 1) / ngpus;
    int64_t lo = (int64_t)rank * S;
    int64_t hi = lo + S;
    if (lo > rows)
        lo = rows;
    if (hi > rows)
        hi = rows;
    *first = lo;
    *count = hi - lo;
}

int64_t oracle_stage_bytes(int64_t rows, int64_t cols, int ngpus, int simd_width)
{
    int64_t S = (rows + ngpus - 1) / ngpus;
    int64_t scale_bytes = S * (int64_t)sizeof(float);
    int64_t padded = (scale_bytes + simd_width - 1) / simd_width * simd_width;
    return S * cols + padded;
}

int oracle_stage_share(const uint8_t *out_fp8, const float *scales, int64_t rows,
                       int64_t cols, int ngpus, int rank, int simd_width, uint8_t *staging)
{
    if (out_fp8 == NULL || scales == NULL || staging == NULL || ngpus < 1 || rank < 0 ||
        rank >= ngpus || rows < 0 || cols <= 0 || simd_width < 1)
        return ORACLE_BAD_ARG;
    int64_t S = (rows + ngpus - 1) / ngpus;
    int64_t first, count;
    oracle_share_rows(rows, ngpus, rank, &first, &count);
    for (int64_t i = 0; i < count; ++i) {
        for (int64_t j = 0; j < cols; ++j)
            staging[i * cols + j] = out_fp8[(first + i) * cols + j];
        memcpy(staging + S * cols + i * (int64_t)sizeof(float), &scales[first + i], sizeof(float));
    }
    return ORACLE_OK;
}
