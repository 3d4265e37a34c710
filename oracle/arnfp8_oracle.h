/*
 * arnfp8_oracle.h -- CPU oracle for the fused all-reduce sum + residual + RMSNorm
 * + per-row dynamic FP8 (e4m3fn) quantisation epilogue.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library.  The GPU product
 * path shares no code, header, table or helper with it.
 *
 * Number formats at this interface:
 *   bf16    -> uint16_t bit patterns
 *   e4m3fn  -> uint8_t  bit patterns (OCP FP8 E4M3, bias 7, max 448, no inf)
 *   e5m2    -> uint8_t  bit patterns (OCP FP8 E5M2, bias 15, max 57344, has inf)
 *   fp32    -> float
 * All tensors are dense row-major [rows, cols]; every call is single-threaded,
 * synchronous, and writes only the outputs it is given.
 */
#ifndef ARNFP8_ORACLE_H
#define ARNFP8_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- number-format codecs --------------------------------------------- */

/* bf16 -> fp32: the bf16 pattern is the upper half of the fp32 pattern. */
float oracle_bf16_to_f32(uint16_t b);

/* fp32 -> bf16, round to nearest, ties to even.  NaN stays NaN (quieted). */
uint16_t oracle_f32_to_bf16(float f);

/* e4m3fn code -> its exact value (NaN for 0x7F / 0xFF). */
double oracle_e4m3fn_to_f64(uint8_t code);

/* fp32 -> e4m3fn: round to nearest, ties to even, saturating at +-448.
 * NaN -> 0x7F. */
uint8_t oracle_f32_to_e4m3fn_sat(float v);

/* e5m2 code -> its exact value (+-inf for 0x7C / 0xFC, NaN above). */
double oracle_e5m2_to_f64(uint8_t code);

/* fp32 -> e5m2: round to nearest, ties to even, saturating at +-57344.
 * NaN -> 0x7E. */
uint8_t oracle_f32_to_e5m2_sat(float v);

/* ---- the operation ------------------------------------------------------ */

/* Status codes returned by the oracle entry points. */
#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_NO_MEMORY 2

/* Rank-order sum: out = bf16_rne(((x_0 + x_1) + x_2) + ... + x_{P-1}) with every
 * add in fp32 and x_p the exact fp32 value of inputs[p].  P in [1, 8]. */
int oracle_sum_bf16(const uint16_t *const *inputs, int P, uint16_t *out,
                    int64_t rows, int64_t cols);

/* The fused epilogue, per row i:
 *   s   = rank-order sum (as oracle_sum_bf16)
 *   h   = bf16_rne(fp32(s) + fp32(residual_in)) if residual_in, else s
 *   residual_out <- h (if residual_out; may equal residual_in)
 *   g_j = fl32(fp32(gamma_j) + weight_offset)
 *   r   = 1 / sqrt(mean_j(h_j^2) + eps), or 0 when mean + eps == 0 (an
 *         all-zero row with eps = 0: y = 0, floor scale, zero codes)  (fp64)
 *   y_j = h_j * r * g_j                                           (fp64)
 *   amax = fl32(max_j |y_j|)
 *   scale = max(min(amax, scale_ub) / 448, 1 / (448 * 512))        (fp32)
 *   q_j = e4m3fn_rne_sat(fl32(y_j / scale))
 * scales[i] = scale.  out_fp8 holds the q codes.
 * eps must be finite and >= 0, weight_offset finite, scale_ub > 0 (+inf: no
 * bound); otherwise ORACLE_BAD_ARG (the MX variant checks eps and the offset). */
int oracle_arnfp8(const uint16_t *const *inputs, int P,
                  const uint16_t *residual_in, uint16_t *residual_out,
                  uint8_t *out_fp8, float *scales, const uint16_t *gamma,
                  float eps, float weight_offset, float scale_ub,
                  int64_t rows, int64_t cols);

/* The same epilogue with e5m2 output: the format maximum 57344 replaces 448,
 *   scale = max(min(amax, scale_ub) / 57344, 1 / (57344 * 512)),
 *   q_j = e5m2_rne_sat(fl32(y_j / scale)). */
int oracle_arnfp8_e5m2(const uint16_t *const *inputs, int P,
                       const uint16_t *residual_in, uint16_t *residual_out,
                       uint8_t *out_fp8, float *scales, const uint16_t *gamma,
                       float eps, float weight_offset, float scale_ub,
                       int64_t rows, int64_t cols);

/* Steps up to the norm only: y [rows, cols] (fp64) = h * r * g, and
 * residual_out as in oracle_arnfp8. */
int oracle_norm_rows(const uint16_t *const *inputs, int P, const uint16_t *residual_in,
                     uint16_t *residual_out, const uint16_t *gamma, float eps,
                     float weight_offset, int64_t rows, int64_t cols, double *y);

/* MXFP8 (OCP MX v1.0, E4M3 elements, blocks of 32, E8M0 scales):
 * shared exponent of a block, floor(log2(max |v|)) - 8 clamped to [-127, 127]
 * (-127 for an all-zero block) ... */
int oracle_mx_shared_exp(const double *v, int n);
/* ... and its codes: e4m3fn_rne_sat(fl32(v * 2^-shared_exp)). */
void oracle_mx_quantize_block(const double *v, int n, int shared_exp, uint8_t *codes);

/* The epilogue with MXFP8 output instead of the per-row scale: out_fp8
 * [rows, cols] e4m3fn, block_scales [rows, cols / 32] E8M0 bytes (e + 127).
 * cols % 32 == 0.  There is no scale_ub: MX scales are not clamped. */
int oracle_arnfp8_mx(const uint16_t *const *inputs, int P,
                     const uint16_t *residual_in, uint16_t *residual_out,
                     uint8_t *out_fp8, uint8_t *block_scales, const uint16_t *gamma,
                     float eps, float weight_offset, int64_t rows, int64_t cols);

/* ---- two-stage row share and its staging layout ------------------------ */
/*
 * In the two-stage (large payload) path each of `ngpus` ranks owns
 * S = ceil(rows / ngpus) consecutive rows: rank k owns [k*S, min(rows, (k+1)*S)).
 * It writes the fp8 rows of its share, then their fp32 scales, into one
 * staging slot:  S * cols bytes of fp8 data, then S * 4 bytes of scales
 * padded up to a multiple of `simd_width` bytes.
 */

/* First row and row count of rank `rank`'s share (count may be 0). */
void oracle_share_rows(int64_t rows, int ngpus, int rank, int64_t *first, int64_t *count);

/* Bytes of one staging slot (fp8 data + padded scales). */
int64_t oracle_stage_bytes(int64_t rows, int64_t cols, int ngpus, int simd_width);

/* Place rank `rank`'s share of a full fused output (out_fp8 [rows, cols],
 * scales [rows]) into `staging` (oracle_stage_bytes bytes; bytes of the slot
 * that the share does not fill are left untouched). */
int oracle_stage_share(const uint8_t *out_fp8, const float *scales, int64_t rows,
                       int64_t cols, int ngpus, int rank, int simd_width, uint8_t *staging);

#ifdef __cplusplus
}
#endif

#endif /* ARNFP8_ORACLE_H */
