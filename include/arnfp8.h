/*
 * arnfp8.h -- C ABI of the MI355X (gfx950) fused all-reduce epilogue library.
 *
 * One GPU holds P per-rank bf16 slabs in HBM, the packs a rank would pull from
 * its peers.  The library sums them in fp32 in rank order and rounds once to
 * bf16, optionally adds a bf16 residual and writes the updated residual back,
 * applies RMSNorm with gain gamma + weight_offset, and quantises every row to
 * fp8 e4m3fn with one dynamic fp32 scale per row -- all in one kernel launch.
 *
 * Sources for the operation:
 *   - Modular Mojo API docs, "allreduce_rmsnorm_fp8" (function summary: the
 *     all-reduce, RMSNorm and FP8 dynamic quantisation happen in a single
 *     launch with no global-memory round trip between the reduction and the
 *     norm; Args: input_buffers, output, gamma, epsilon, weight_offset,
 *     scale_ub, scale_output).
 *   - b12x PR #283 "PCIeTwoShotBF16" (PR description: fp32 accumulation in a
 *     fixed rank order, one rounding to bf16, deterministic across calls and
 *     graph replays).
 *   - TensorRT-LLM PR #19836 (Description: the RESIDUAL_RMS_NORM epilogue --
 *     residual add, residual write-back, RMSNorm).
 *   - tt-metal rmsnorm_2d.py (RMSNorm2DConfig.add_unit_offset: gain 1 + gamma).
 *
 * Conventions shared by every entry point
 *   - Every tensor is dense row-major, with no strides.  bf16 and fp8 tensors
 *     are passed as untyped device pointers; fp32 tensors as float*.
 *   - Device pointers must be 16-byte aligned (the kernels move 16-byte
 *     vectors), except `scales`, which must be 4-byte aligned.
 *   - `cols` must be a positive multiple of 8 and at most ARNFP8_MAX_COLS;
 *     `rows` may be 0 (the call then does nothing and returns ARNFP8_OK).
 *   - 1 <= P <= ARNFP8_MAX_P.  The host array `inputs` is read during the call
 *     and its P pointers are passed by value to the kernel; the caller may
 *     reuse the array as soon as the call returns.
 *   - Ownership: the caller owns every buffer.  The library allocates nothing
 *     and keeps no state between calls beyond a cached compute-unit count per
 *     device and the split path's per-row counts (in the caller's workspace,
 *     or in the library's own array for arnfp8_run_split_noalloc), so calls
 *     may be captured in a HIP graph; pointers captured that way must stay
 *     valid for the graph's life.
 *   - Validation happens on the host before any launch and touches no device
 *     state; a call that returns an error has launched nothing.
 *   - Execution is asynchronous on `stream` (NULL = the default stream);
 *     results are visible to later work on that stream.  Results are
 *     deterministic: bitwise identical on every call with the same arguments
 *     (the automatic launch shape depends only on rows, cols, P and the
 *     device), including calls replayed from a captured graph.
 *   - Concurrent calls on different streams must not share output buffers
 *     (nor, on the split path, a workspace).
 *   - Non-finite inputs are not supported (the results are unspecified), nor
 *     are rows whose sum of squares leaves the fp32 range (|h| of order 1e18
 *     and above): the row statistics are fp32.
 */
#ifndef ARNFP8_H
#define ARNFP8_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ARNFP8_MAX_P 8
#define ARNFP8_MAX_COLS 65536

/*
 * Status codes.  Every entry point returns one; all of them except
 * ARNFP8_HIP_ERROR are decided on the host before anything is launched.
 * Returning a status code from a first phase that validates the arguments is
 * the convention of Huawei CANN aclnnAlltoAllQuantMatmul (Returns: a status
 * code; the first-phase API validates the input parameters).  The checks
 * themselves are the ones b12x PR #283 "PCIeTwoShotBF16" is asked to make in
 * review: payload and caller-provided output tensors checked for alignment,
 * shape and capacity before any device launch, so that no launch reads
 * misaligned data or writes out of bounds.
 */
#define ARNFP8_OK 0
/* A required pointer is NULL.  CANN aclnnAlltoAllQuantMatmul (constraints:
 * the inputs and the output are not null pointers). */
#define ARNFP8_NULL_POINTER 1
/* A pointer breaks the alignment rule above.  b12x PR #283 review (the payload
 * must be 16-byte aligned, as the kernel's vector loads assume; misaligned
 * tensors are rejected before launch). */
#define ARNFP8_MISALIGNED 2
/* rows < 0, cols <= 0, cols % 8, cols > ARNFP8_MAX_COLS, or the byte size
 * overflows int64.  b12x PR #283 (Behavior: accepts() rejects a tensor whose
 * size does not fit the row width or exceeds the row capacity; Validation:
 * rejections by dtype, row width, row count and capacity are tested); CANN
 * aclnnAlltoAllQuantMatmul (constraints: upper and lower bounds on the
 * sizes). */
#define ARNFP8_BAD_SHAPE 3
/* P outside [1, ARNFP8_MAX_P].  Mojo docs "allreduce_rmsnorm_fp8" (rank_sigs:
 * 8 signal slots, so at most 8 ranks); b12x PR #283 (world sizes 2, 4, 8). */
#define ARNFP8_BAD_P 4
/* An output overlaps an input or another output (residual_out == residual_in
 * is allowed).  b12x PR #283 review (caller-provided output tensors are
 * validated before their pointers reach device code, to prevent incorrect
 * writes). */
#define ARNFP8_ALIAS 5
/* The kernel launch call itself failed (the HIP runtime's error). */
#define ARNFP8_HIP_ERROR 6
/* An arnfp8_run_ex launch option is invalid (this library's own tuning
 * interface; no page defines it). */
#define ARNFP8_BAD_CONFIG 7
/* ngpus < 1, or rank outside [0, ngpus).  Mojo docs "allreduce_rmsnorm_fp8"
 * (the 2-stage path: ngpus ranks, each owning ceildiv(rows, ngpus) rows). */
#define ARNFP8_BAD_SHARE 8
/* Unknown out_format.  CANN aclnnAlltoAllQuantMatmul (x1QuantDtype and the
 * quantisation modes name the supported output types). */
#define ARNFP8_BAD_FORMAT 9
/* eps NaN, infinite or negative; weight_offset NaN or infinite; or, for the
 * per-row formats, scale_ub NaN or <= 0 (+inf is allowed: no upper bound).
 * Mojo docs "allreduce_rmsnorm_fp8" (Args: epsilon is the RMSNorm's
 * stabilising term, weight_offset an additive offset of gamma, scale_ub the
 * upper bound of the scale clamp). */
#define ARNFP8_BAD_SCALAR 10
/* The split workspace is missing space: fewer than
 * arnfp8_split_workspace_bytes(rows) bytes for arnfp8_run_split, more than
 * ARNFP8_NOALLOC_MAX_ROWS rows for arnfp8_run_split_noalloc (this library's
 * own interface). */
#define ARNFP8_BAD_WORKSPACE 11

/*
 * arnfp8_run -- the fused epilogue.  For every row i and column j:
 *   s    = bf16_rne(((x_0 + x_1) + ...) + x_{P-1}),   x_p = fp32(inputs[p][i,j]),
 *          every add in fp32, in rank order (rank 0's value starts the sum)
 *   h    = bf16_rne(fp32(s) + fp32(residual_in[i,j]))  if residual_in, else s
 *   residual_out[i,j] = h                               if residual_out
 *   g_j  = fp32(gamma[j]) + weight_offset                          (fp32)
 *   r    = 1 / sqrt(sum_j h_j^2 / cols + eps)   (0 if that sum is 0: see eps)
 *   amax = max_j |h_j * g_j| * r
 *   scale = max(min(amax, scale_ub) / 448, 1 / (448 * 512))
 *   out_fp8[i,j] = e4m3fn(clamp(h_j * g_j * r / scale, -448, 448)),
 *          round to nearest even;  scales[i] = scale.
 *
 * inputs       host array of P device pointers, bf16 [rows, cols], rank order
 * residual_in  device bf16 [rows, cols], or NULL (no residual add)
 * residual_out device bf16 [rows, cols], or NULL; may equal residual_in
 *              (in-place update).  With residual_in == NULL it receives s.
 * out_fp8      device e4m3fn [rows, cols] (OCP FP8 E4M3: bias 7, max 448)
 * scales       device fp32 [rows] (the [rows, 1] per-row scales)
 * gamma        device bf16 [cols]
 * eps          fp32, finite and >= 0.  With eps = 0 a row whose mean square is
 *              0 (all h zero) has nothing to normalise: r is taken as 0, so
 *              the row gets the floor scale and zero codes (never a NaN code).
 *              The mean square is fp32 here, so with eps = 0 a row whose
 *              mean square is not a normal fp32 number (RMS below about
 *              1e-19) lies outside the supported range, like rows whose
 *              sum of squares overflows.
 * weight_offset fp32, finite.
 * scale_ub     fp32, > 0 (+inf: no upper bound).
 *              Any other eps, weight_offset or scale_ub: ARNFP8_BAD_SCALAR.
 * Norm and scale arithmetic is fp32.  r comes from the hardware reciprocal
 * square root of fl32(sum_j h_j^2 * fl32(1 / cols)) + eps, and 1 / scale from
 * the hardware reciprocal (each within 1 ulp); the division by 448 is IEEE, so
 * a clamped scale is exactly fl32(scale_ub / 448).  Scales agree with the
 * exact definition to within a few fp32 ulps.
 */
int arnfp8_run(const void *const *inputs, const void *residual_in, void *residual_out,
               void *out_fp8, float *scales, const void *gamma, float eps,
               float weight_offset, float scale_ub, int64_t rows, int64_t cols, int P,
               hipStream_t stream);

/* Kernel variants selectable through arnfp8_launch.variant. */
#define ARNFP8_VARIANT_AUTO 0 /* the library's choice from (rows, cols, P)        */
#define ARNFP8_VARIANT_ROW 1  /* one workgroup per row, rows walked grid-stride  */

/* Cache policy of the fused kernel's row outputs (arnfp8_launch.stores).  nt
 * is the fastest when the output buffers are not cache-resident between calls;
 * sc1 is faster only when the same buffers are rewritten while still cached.
 * The policy never changes a result. */
#define ARNFP8_STORES_AUTO 0 /* the library's choice: currently nt            */
#define ARNFP8_STORES_NT 1   /* non-temporal stores                          */
#define ARNFP8_STORES_SC1 2  /* device-scope coherent (sc1) stores           */

/* Launch options for arnfp8_run_ex / arnfp8_run_fmt.  Zero in any field means
 * "automatic".  No option changes a bf16 result (see arnfp8_run_ex for the
 * last bits of scales and fp8 codes). */
typedef struct arnfp8_launch {
  int variant; /* ARNFP8_VARIANT_*                                               */
  int threads; /* lanes per workgroup: a multiple of 64 in [64, 512], or up to
                  1024 with one chunk per lane (vpt 1)                          */
  int vpt;     /* 16-byte chunks per lane: 1, 2, 4, 8 or 16                    */
  int grid;    /* workgroups; rows are walked grid-stride (>= 1); grid * threads
                  must fit in 32 bits                                           */
  int stores;  /* ARNFP8_STORES_*                                               */
} arnfp8_launch;

/*
 * arnfp8_run_ex -- arnfp8_run with explicit launch options (for tuning and for
 * testing every kernel shape).  `opt` may be NULL (= arnfp8_run).  The options
 * must satisfy threads * vpt * 8 >= cols; otherwise, or for an out-of-range
 * field, the call returns ARNFP8_BAD_CONFIG without launching.  bf16 outputs
 * do not depend on the options; fp32 scales and fp8 codes may differ in the
 * last bits between launch shapes (the sum of squares is reduced in a
 * shape-dependent order), each staying within the operation's tolerance.
 */
int arnfp8_run_ex(const void *const *inputs, const void *residual_in, void *residual_out,
                  void *out_fp8, float *scales, const void *gamma, float eps,
                  float weight_offset, float scale_ub, int64_t rows, int64_t cols, int P,
                  hipStream_t stream, const arnfp8_launch *opt);

/* Output formats for arnfp8_run_fmt. */
#define ARNFP8_FMT_E4M3FN 0 /* OCP e4m3fn, one fp32 scale per row (arnfp8_run)      */
#define ARNFP8_FMT_E5M2 1   /* OCP e5m2, one fp32 scale per row                      */
#define ARNFP8_FMT_MXFP8 2  /* OCP MXFP8: e4m3fn, one E8M0 scale per 32 values       */

/*
 * arnfp8_run_fmt -- the fused epilogue with a choice of quantised output.
 * Per-token dynamic quantisation to E4M3FN or E5M2 and the mx (microscaling)
 * mode are the quantisation variants of Huawei CANN aclnnAlltoAllQuantMatmul
 * (x1QuantMode, x1QuantDtype; the mx scale shape (BS, ceil(H/64), 2)).
 *   ARNFP8_FMT_E4M3FN  as arnfp8_run.
 *   ARNFP8_FMT_E5M2    as arnfp8_run with the e5m2 maximum 57344 in place of
 *                      448: scale = max(min(amax, scale_ub) / 57344,
 *                      1 / (57344 * 512)); out_fp8 holds OCP e5m2 codes.
 *   ARNFP8_FMT_MXFP8   no per-row scale and no scale_ub (ignored, not
 *                      validated): every block
 *                      of 32 consecutive values of a row gets the shared
 *                      exponent e = floor(log2(max |y|)) - 8, clamped to
 *                      [-127, 127] (-127 for an all-zero block), and its values
 *                      are e4m3fn(clamp(y * 2^-e, -448, 448)), y = h * g * r;
 *                      `scales` is uint8 [rows, cols / 32] holding e + 127
 *                      (E8M0), the (rows, cols / 64, 2) layout when cols % 64
 *                      == 0.  Requires cols % 32 == 0 (else ARNFP8_BAD_SHAPE).
 *                      Rule: OCP Microscaling Formats v1.0 (MXFP8 E4M3).
 * `scales` is float* for the per-row formats (4-byte aligned) and uint8_t*
 * for MXFP8.  `opt` as for arnfp8_run_ex (may be NULL).  An unknown
 * out_format returns ARNFP8_BAD_FORMAT.
 */
int arnfp8_run_fmt(const void *const *inputs, const void *residual_in, void *residual_out,
                   void *out_fp8, void *scales, const void *gamma, float eps,
                   float weight_offset, float scale_ub, int64_t rows, int64_t cols, int P,
                   int out_format, hipStream_t stream, const arnfp8_launch *opt);

/*
 * Split rows (small batches and one token).  TensorRT-LLM PR #19836
 * (Description) spreads a one-token row of the RESIDUAL_RMS_NORM epilogue over
 * a cluster of 8 CTAs that trade partial sums.  arnfp8_run_split spreads each
 * row over `parts` workgroups the same way, so that a row's bytes stream into
 * several compute units at once; the parts trade their partial (sum h^2,
 * max |h g|) through `workspace`, one relaxed 64-bit atomic word per value,
 * and wait for one another (boundedly).
 *
 * The result is that of arnfp8_run (e4m3fn output) for the same arguments,
 * within the operation's tolerance: bf16 outputs are identical, scales and
 * codes may differ in the last bits, as between launch shapes (the sum of
 * squares is reduced per part, then over the parts in order).  Results are
 * deterministic, also when a part runs out of waiting: it then computes the
 * late partner's partial itself, from the inputs, bitwise as the partner does.
 * For that reason residual_out must not be residual_in (ARNFP8_ALIAS): the
 * late partner's residual input must still be there to be read.  With one
 * part per row (asked for, or the automatic choice at larger batches and for
 * rows under 128 chunks) there is nothing to trade: the call launches
 * arnfp8_run's kernel in arnfp8_run's launch shape, with the same result
 * bits, and leaves the workspace as it is.
 *
 * workspace  device memory of at least arnfp8_split_workspace_bytes(rows)
 *            bytes, 16-byte aligned, overlapping no input or output, set to
 *            zero before its first use and then left to the library (it
 *            keeps per-row counts between calls; any later call of any shape
 *            may use it).  Calls that may run at the same time (other
 *            streams) need workspaces of their own.  Else ARNFP8_NULL_POINTER,
 *            ARNFP8_MISALIGNED, ARNFP8_BAD_WORKSPACE or ARNFP8_ALIAS.
 * opt        NULL for the automatic choice, else:
 *   parts      workgroups per row, 1..8 (0: the largest power of two up to 8
 *              with rows * parts <= the compute units and at least 64 chunks
 *              of 16 bytes per part, at least 1); a part holds
 *              ceil(cols / 8 / parts) chunks, at most 1024 (else
 *              ARNFP8_BAD_CONFIG)
 *   spin_polls polls of a partner's words before its partial is computed
 *              locally: 0 for the default (32768), -1 for none at once (the
 *              fallback alone, for testing), else the count
 * Every other argument and rule is that of arnfp8_run.
 */
typedef struct arnfp8_split_opts {
  int parts;
  int spin_polls;
} arnfp8_split_opts;

/* The parts per row arnfp8_run_split picks when opt is NULL or opt->parts is 0,
 * on the current device (its compute-unit count), for rows x cols: 1..8, or -1
 * when rows <= 0 or cols is not a valid width.  Queries the device only for
 * its compute-unit count (256 is assumed when no device can be queried). */
int arnfp8_split_parts(int64_t rows, int64_t cols);

/* Workspace bytes arnfp8_run_split needs for `rows` rows (128 per row), or -1
 * for rows < 0. */
int64_t arnfp8_split_workspace_bytes(int64_t rows);

int arnfp8_run_split(const void *const *inputs, const void *residual_in, void *residual_out,
                     void *out_fp8, float *scales, const void *gamma, float eps,
                     float weight_offset, float scale_ub, int64_t rows, int64_t cols, int P,
                     void *workspace, int64_t workspace_bytes, hipStream_t stream,
                     const arnfp8_split_opts *opt);

/*
 * arnfp8_run_split_noalloc -- arnfp8_run_split for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It allocates nothing and takes no
 * workspace: the workspace is a device array of this library, 128 bytes per
 * row for up to ARNFP8_NOALLOC_MAX_ROWS rows (512 KiB), which every device
 * the library runs on holds until the process ends.
 *
 *   rows       at most ARNFP8_NOALLOC_MAX_ROWS, else ARNFP8_BAD_WORKSPACE
 *              (checked after the shape, before everything else)
 *   stream     a stream of the current device; the array used is that
 *              device's.  Every argument is validated first (no workspace
 *              checks apply); the first call on a device that launches the
 *              split kernel then looks the array's address up and clears the
 *              array on `stream`, before its own launch.  A call with one part
 *              per row runs arnfp8_run's kernel and does not use the array.
 * Every call on a device shares that device's array and leaves its per-row
 * counts for the next call, of any shape: calls that may run at the same time
 * on one device (other streams, other threads) race and give wrong results;
 * order them (one stream, or events).  Every other argument, rule and status
 * is that of arnfp8_run_split, whose kernels it launches; outputs are bitwise
 * those of arnfp8_run_split with the same arguments and options.
 */
#define ARNFP8_NOALLOC_MAX_ROWS 4096

int arnfp8_run_split_noalloc(const void *const *inputs, const void *residual_in,
                             void *residual_out, void *out_fp8, float *scales, const void *gamma,
                             float eps, float weight_offset, float scale_ub, int64_t rows,
                             int64_t cols, int P, hipStream_t stream,
                             const arnfp8_split_opts *opt);

/*
 * arn_sum_bf16 -- the reduction alone: out = s as defined for arnfp8_run.
 * out is device bf16 [rows, cols] and must not overlap any input.
 * Source: b12x PR #283 "PCIeTwoShotBF16" (PR description).
 */
int arn_sum_bf16(const void *const *inputs, void *out, int64_t rows, int64_t cols, int P,
                 hipStream_t stream);

/*
 * Two-stage (large payload) row share.  With `ngpus` ranks each rank owns
 * S = ceil(rows / ngpus) consecutive rows, rank k the rows [k*S, min(rows,
 * (k+1)*S)) (possibly none).  It reduces and normalises only its share and
 * writes the share's fp8 rows and scales into one staging slot, from which the
 * other ranks gather it:
 *   bytes [0, S*cols)                        fp8 e4m3fn rows of the share
 *   bytes [S*cols, S*cols + S*4)             fp32 scales of the share
 *   padded to ARNFP8_SIMD_WIDTH              (slot size: arnfp8_stage_bytes)
 * Source: Modular Mojo API docs, "allreduce_rmsnorm_fp8" (2-stage path:
 * signal buffer sizing of ceildiv(rows, ngpus) * cols fp8 bytes plus the
 * scales aligned up to the SIMD width; the signal header is not part of the
 * slot here).  Rows past the share's end in a shorter last share leave their
 * slot bytes untouched.
 */
#define ARNFP8_SIMD_WIDTH 16

/* Bytes of one staging slot, or -1 for rows < 0, cols <= 0, ngpus < 1. */
int64_t arnfp8_stage_bytes(int64_t rows, int64_t cols, int ngpus);

/*
 * arnfp8_run_share -- arnfp8_run restricted to rank `rank`'s share.
 * inputs, residual_in, residual_out are the full [rows, cols] tensors; only
 * the share's rows are read, and only the share's rows of residual_out are
 * written.  staging is device memory of arnfp8_stage_bytes(rows, cols, ngpus)
 * bytes, 16-byte aligned, overlapping no input or residual_out.  Every other
 * argument and rule is that of arnfp8_run.  An empty share returns ARNFP8_OK
 * after validation and launches nothing.
 */
int arnfp8_run_share(const void *const *inputs, const void *residual_in, void *residual_out,
                     void *staging, const void *gamma, float eps, float weight_offset,
                     float scale_ub, int64_t rows, int64_t cols, int P, int ngpus, int rank,
                     hipStream_t stream);

/*
 * arnfp8_convert_f32 -- the kernels' number-format conversion step on its own
 * (for checking the hardware conversion instructions exhaustively).
 *   ARNFP8_FMT_E4M3FN  out = e4m3fn(clamp(in, -448, 448)),     1 byte each
 *   ARNFP8_FMT_E5M2    out = e5m2(clamp(in, -57344, 57344)),   1 byte each
 *   ARNFP8_CVT_BF16    out = bf16(in),                          2 bytes each
 * all round to nearest even.  in: device fp32 [n]; out: device [n] of the
 * format; n % 8 == 0; both 16-byte aligned and not overlapping.  NaN inputs
 * give unspecified codes.  Returns ARNFP8_BAD_FORMAT for any other format.
 */
#define ARNFP8_CVT_BF16 16
int arnfp8_convert_f32(const float *in, void *out, int64_t n, int format, hipStream_t stream);

/* Human-readable text for a status code (a static string; never NULL; "unknown
 * status" for a code not listed above).  The text of each code restates the
 * rule whose source is cited at the code's definition. */
const char *arnfp8_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ARNFP8_H */
