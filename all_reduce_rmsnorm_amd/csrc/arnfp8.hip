// arnfp8.hip -- the C ABI of the fused all-reduce epilogue library for gfx950:
// argument validation (on the host, before any device query or launch),
// the automatic launch shape, and the launches.  The device code is in
// arnfp8_kernels.hpp; the row kernel's instances are built per output format
// in arnfp8_rows_*.hip.
//
// Sources: Modular Mojo API docs "allreduce_rmsnorm_fp8" (function summary,
// Args; the 2-stage signal buffer sizing); b12x PR #283 "PCIeTwoShotBF16" (PR
// description; the validation the review asks for: alignment, output
// tensors checked before any launch); Huawei CANN aclnnAlltoAllQuantMatmul
// (output formats).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cfloat>
#include <mutex>

#include "arnfp8.h"
#include "arnfp8_kernels.hpp"
#include "arnfp8_tables.hpp"

namespace {

using namespace arnfp8;

// ------------------------------------------------------------ host side ----

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned(const void *p, uintptr_t n) { return ((uintptr_t)p % n) == 0; }

int check_shape(int64_t rows, int64_t cols, int P) {
  if (P < 1 || P > ARNFP8_MAX_P) return ARNFP8_BAD_P;
  if (rows < 0 || cols <= 0 || cols % 8 != 0 || cols > ARNFP8_MAX_COLS) return ARNFP8_BAD_SHAPE;
  if (rows > INT64_MAX / (2 * cols)) return ARNFP8_BAD_SHAPE;
  return ARNFP8_OK;
}

// The norm's scalars: eps finite and >= 0, weight_offset finite, and (for the
// per-row formats) scale_ub > 0, +inf meaning no bound.  NaN fails every
// comparison below, so it is rejected too.
int check_scalars(float eps, float weight_offset, float scale_ub, bool check_ub) {
  if (!(eps >= 0.0f && eps <= FLT_MAX) || !(weight_offset >= -FLT_MAX && weight_offset <= FLT_MAX))
    return ARNFP8_BAD_SCALAR;
  if (check_ub && !(scale_ub > 0.0f)) return ARNFP8_BAD_SCALAR;
  return ARNFP8_OK;
}

int check_inputs(const void *const *inputs, int P) {
  if (inputs == nullptr) return ARNFP8_NULL_POINTER;
  for (int p = 0; p < P; ++p)
    if (inputs[p] == nullptr) return ARNFP8_NULL_POINTER;
  for (int p = 0; p < P; ++p)
    if (!aligned(inputs[p], 16)) return ARNFP8_MISALIGNED;
  return ARNFP8_OK;
}

// Launches `kernel` with its arguments passed by value; the status is that of
// this launch alone (not an earlier error left in the thread's HIP state).
template <typename... Args>
int launch(void (*kernel)(Args...), dim3 grid, dim3 block, hipStream_t stream, Args... args) {
  void *argv[] = {(void *)&args...};
  return hipLaunchKernel((const void *)kernel, grid, block, argv, 0, stream) == hipSuccess
             ? ARNFP8_OK
             : ARNFP8_HIP_ERROR;
}

// Compute units of the current device (queried once per device).
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// ---- launch tables: one entry per template instance ----

typedef void (*SumKernel)(Slabs, u32x4 *, int64_t);

template <int U>
SumKernel sum_kernel_p(int P) {
  switch (P) {
    case 1: return arn_sum_kernel<1, U>;
    case 2: return arn_sum_kernel<2, U>;
    case 3: return arn_sum_kernel<3, U>;
    case 4: return arn_sum_kernel<4, U>;
    case 5: return arn_sum_kernel<5, U>;
    case 6: return arn_sum_kernel<6, U>;
    case 7: return arn_sum_kernel<7, U>;
    default: return arn_sum_kernel<8, U>;
  }
}

RowKernel row_table(int fmt, int P, int vpt, bool res_in, bool res_out, bool sc1) {
  switch (fmt) {
    case ARNFP8_FMT_E5M2: return row_table_e5m2(P, vpt, res_in, res_out, sc1);
    case ARNFP8_FMT_MXFP8: return row_table_mxfp8(P, vpt, res_in, res_out, sc1);
    default: return row_table_e4m3(P, vpt, res_in, res_out, sc1);
  }
}

struct RowConfig {
  int threads;
  int vpt;
  int grid;
  int sc1_stores;
};

// Smallest chunks-per-lane (1, 2, 4, 8, 16) that fits the row in at most 512
// lanes.  Lanes are rounded up to whole waves, except that batches smaller
// than 32 rows per CU use all 512 lanes when a lane holds two or more
// chunks.  Measured on MI355X for 7168-wide rows, P = 8, inputs out of
// cache, graph replay: 512 x 2 against 448 x 2 is 9.78 / 9.90 us at 256 rows,
// 28.5 / 28.9 us at 1024, 54.1 / 55.9 us at 2048, 104.0 / 104.7 us at 4096
// and 178.2 / 179.2 us at 7168; at 8192 rows the two are level under graph
// replay and 448 x 2 is ~1 % faster back to back.  Four chunks per lane (256
// lanes, also with four workgroups per CU resident) and one (896 lanes) are
// slower at every batch from 256 rows up.  Row outputs use nt stores (the
// fastest policy when the output buffers are not cache-resident, at every
// batch size measured).
// With eight slabs and at most one row per CU, one chunk per lane (up to 1024
// lanes) is faster: measured (graph replay, inputs out of cache / the same
// inputs every call) at 1 row 5.71 / 3.75 against 5.89 / 3.90 us for
// 7168-wide rows and 5.84 / 3.75 against 6.08 / 3.89 us for 8192-wide rows,
// and 2-3 % faster out of cache up to 256 rows.  With four slabs (7168
// columns) it trades: 0.1-0.25 us faster out of cache and 0.08-0.16 us
// slower with the inputs cache-warm, from 1 to 128 rows (32 rows: 5.26 /
// 3.49 against 5.35 / 3.40 us); two chunks per lane are kept there.
RowConfig pick_row_config(int64_t rows, int c16, int P) {
  static const int vpts[5] = {1, 2, 4, 8, 16};
  const int64_t cus = device_cus();
  const bool small_batch = rows < 32 * cus;
  RowConfig cfg{512, 16, 1, 0};
  if (P >= 8 && rows <= cus && c16 <= 1024) {
    cfg.vpt = 1;
    cfg.threads = (c16 + 63) / 64 * 64;
    cfg.grid = (int)rows;
    return cfg;
  }
  for (int i = 0; i < 5; ++i) {
    const int lanes = (c16 + vpts[i] - 1) / vpts[i];
    if (lanes <= 512) {
      cfg.vpt = vpts[i];
      cfg.threads = (vpts[i] > 1 && small_batch) ? 512 : ((lanes + 63) / 64) * 64;
      break;
    }
  }
  cfg.grid = (int)(rows < 65536 ? rows : 65536);
  return cfg;
}

// Validates the fused call's arguments and fills the kernel arguments.
int prepare_fused(const void *const *inputs, const void *residual_in, void *residual_out,
                  void *out_fp8, void *scales, const void *gamma, float eps,
                  float weight_offset, float scale_ub, int64_t rows, int64_t cols, int P,
                  RowArgs *a, int fmt = ARNFP8_FMT_E4M3FN) {
  int st = check_inputs(inputs, P);
  if (st != ARNFP8_OK) return st;
  if (out_fp8 == nullptr || scales == nullptr || gamma == nullptr) return ARNFP8_NULL_POINTER;
  if (!aligned(out_fp8, 16) || !aligned(gamma, 16) ||
      !aligned(scales, fmt == ARNFP8_FMT_MXFP8 ? 1 : 4) ||
      (residual_in && !aligned(residual_in, 16)) || (residual_out && !aligned(residual_out, 16)))
    return ARNFP8_MISALIGNED;

  // No output may overlap an input or another output; the one exception is
  // residual_out == residual_in exactly (the in-place residual update).
  const uintptr_t n = (uintptr_t)(rows * cols);
  Range ins[ARNFP8_MAX_P + 2];
  int nin = 0;
  for (int p = 0; p < P; ++p) ins[nin++] = Range{(uintptr_t)inputs[p], (uintptr_t)inputs[p] + 2 * n};
  ins[nin++] = Range{(uintptr_t)gamma, (uintptr_t)gamma + 2 * (uintptr_t)cols};
  const int res_in_slot = residual_in ? nin : -1;
  if (residual_in) ins[nin++] = Range{(uintptr_t)residual_in, (uintptr_t)residual_in + 2 * n};
  Range outs[3];
  int nout = 0;
  outs[nout++] = Range{(uintptr_t)out_fp8, (uintptr_t)out_fp8 + n};
  const uintptr_t scale_bytes =
      fmt == ARNFP8_FMT_MXFP8 ? (uintptr_t)(rows * (cols / 32)) : 4 * (uintptr_t)rows;
  outs[nout++] = Range{(uintptr_t)scales, (uintptr_t)scales + scale_bytes};
  const int res_out_slot = residual_out ? nout : -1;
  if (residual_out) outs[nout++] = Range{(uintptr_t)residual_out, (uintptr_t)residual_out + 2 * n};
  for (int o = 0; o < nout; ++o) {
    for (int i = 0; i < nin; ++i) {
      const bool in_place = o == res_out_slot && i == res_in_slot && residual_out == residual_in;
      if (!in_place && overlaps(outs[o], ins[i])) return ARNFP8_ALIAS;
    }
    for (int o2 = o + 1; o2 < nout; ++o2)
      if (overlaps(outs[o], outs[o2])) return ARNFP8_ALIAS;
  }

  for (int p = 0; p < ARNFP8_MAX_P; ++p) a->in.p[p] = (const u32x4 *)inputs[p < P ? p : 0];
  a->res_in = (const u32x4 *)residual_in;
  a->res_out = (u32x4 *)residual_out;
  a->out = (u32x2 *)out_fp8;
  a->scales = fmt == ARNFP8_FMT_MXFP8 ? nullptr : (float *)scales;
  a->mx_scales = fmt == ARNFP8_FMT_MXFP8 ? (uint8_t *)scales : nullptr;
  a->gamma = (const u32x4 *)gamma;
  a->eps = eps;
  a->woff = weight_offset;
  a->ub = scale_ub;
  a->inv_cols = 1.0f / (float)cols;
  a->rows = rows;
  a->c16 = (int)(cols / 8);
  return ARNFP8_OK;
}

// Resolves the launch options against the automatic choice.  The options are
// checked first; the device is queried only when lanes and chunks per lane
// are both left automatic.
int resolve_row_config(const arnfp8_launch *opt, int64_t rows, int c16, int P, RowConfig *cfg) {
  static const int vpts[5] = {1, 2, 4, 8, 16};
  if (opt == nullptr) {
    *cfg = pick_row_config(rows, c16, P);
    return ARNFP8_OK;
  }
  if (opt->variant != ARNFP8_VARIANT_AUTO && opt->variant != ARNFP8_VARIANT_ROW)
    return ARNFP8_BAD_CONFIG;
  if (opt->stores != ARNFP8_STORES_AUTO && opt->stores != ARNFP8_STORES_NT &&
      opt->stores != ARNFP8_STORES_SC1)
    return ARNFP8_BAD_CONFIG;
  if (opt->threads < 0 || opt->vpt < 0 || opt->grid < 0) return ARNFP8_BAD_CONFIG;
  if (opt->threads && (opt->threads % 64 != 0 || opt->threads > 1024)) return ARNFP8_BAD_CONFIG;
  if (opt->vpt && opt->vpt != 1 && opt->vpt != 2 && opt->vpt != 4 && opt->vpt != 8 &&
      opt->vpt != 16)
    return ARNFP8_BAD_CONFIG;
  if (opt->threads && opt->vpt) {
    cfg->threads = opt->threads;
    cfg->vpt = opt->vpt;
  } else if (opt->threads) {  // the smallest chunks-per-lane that covers the row
    cfg->threads = opt->threads;
    cfg->vpt = 0;
    for (int i = 0; i < 5 && !cfg->vpt; ++i)
      if ((int64_t)vpts[i] * cfg->threads >= c16) cfg->vpt = vpts[i];
    if (!cfg->vpt) return ARNFP8_BAD_CONFIG;
  } else if (opt->vpt) {  // the lanes that cover the row, in whole waves
    cfg->vpt = opt->vpt;
    cfg->threads = ((c16 + cfg->vpt - 1) / cfg->vpt + 63) / 64 * 64;
  } else {
    *cfg = pick_row_config(rows, c16, P);
  }
  // One chunk per lane allows up to 1024 lanes; more chunks per lane, 512.
  if (cfg->threads > (cfg->vpt == 1 ? 1024 : 512)) return ARNFP8_BAD_CONFIG;
  if ((int64_t)cfg->threads * cfg->vpt < c16) return ARNFP8_BAD_CONFIG;
  cfg->grid = opt->grid ? opt->grid : (int)(rows < 65536 ? rows : 65536);
  // A dispatch counts its work-items in 32 bits.
  if ((int64_t)cfg->grid * cfg->threads > (int64_t)UINT32_MAX) return ARNFP8_BAD_CONFIG;
  cfg->sc1_stores = opt->stores == ARNFP8_STORES_SC1;
  return ARNFP8_OK;
}

}  // namespace

// ------------------------------------------------------------------ C ABI --

extern "C" int arn_sum_bf16(const void *const *inputs, void *out, int64_t rows, int64_t cols,
                            int P, hipStream_t stream) {
  int st = check_shape(rows, cols, P);
  if (st != ARNFP8_OK) return st;
  if (rows == 0) return ARNFP8_OK;
  st = check_inputs(inputs, P);
  if (st != ARNFP8_OK) return st;
  if (out == nullptr) return ARNFP8_NULL_POINTER;
  if (!aligned(out, 16)) return ARNFP8_MISALIGNED;
  const uintptr_t bytes = (uintptr_t)(rows * cols * 2);
  const Range o{(uintptr_t)out, (uintptr_t)out + bytes};
  for (int p = 0; p < P; ++p)
    if (overlaps(o, Range{(uintptr_t)inputs[p], (uintptr_t)inputs[p] + bytes})) return ARNFP8_ALIAS;

  Slabs s;
  for (int p = 0; p < ARNFP8_MAX_P; ++p) s.p[p] = (const u32x4 *)inputs[p < P ? p : 0];
  const int64_t n16 = rows * cols / 8;
  // 256 lanes; 4 chunks per lane per iteration once that still gives every CU
  // four workgroups, else 1 (more workgroups for small tensors).  The grid is
  // capped at 16 workgroups per CU.  Measured on MI355X: P = 8 over 8192 x 7168
  // 173 us with 4 chunks vs 185 us with 2; P = 4 over 64 x 4096 1.90 us with 1
  // vs 1.96 us with 2.
  const int threads = 256;
  const int64_t cus = device_cus();
  const bool wide = (n16 + threads * 4 - 1) / (threads * 4) >= 4 * cus;
  const int U = wide ? 4 : 1;
  int64_t blocks = (n16 + threads * U - 1) / (threads * U);
  if (blocks > 16 * cus) blocks = 16 * cus;
  return launch(wide ? sum_kernel_p<4>(P) : sum_kernel_p<1>(P), dim3((unsigned)blocks),
                dim3(threads), stream, s, (u32x4 *)out, n16);
}

extern "C" int arnfp8_run_fmt(const void *const *inputs, const void *residual_in,
                              void *residual_out, void *out_fp8, void *scales, const void *gamma,
                              float eps, float weight_offset, float scale_ub, int64_t rows,
                              int64_t cols, int P, int out_format, hipStream_t stream,
                              const arnfp8_launch *opt) {
  int st = check_shape(rows, cols, P);
  if (st != ARNFP8_OK) return st;
  if (out_format != ARNFP8_FMT_E4M3FN && out_format != ARNFP8_FMT_E5M2 &&
      out_format != ARNFP8_FMT_MXFP8)
    return ARNFP8_BAD_FORMAT;
  if (out_format == ARNFP8_FMT_MXFP8 && cols % 32 != 0) return ARNFP8_BAD_SHAPE;
  st = check_scalars(eps, weight_offset, scale_ub, out_format != ARNFP8_FMT_MXFP8);
  if (st != ARNFP8_OK) return st;
  if (rows == 0) return ARNFP8_OK;
  RowArgs a;
  st = prepare_fused(inputs, residual_in, residual_out, out_fp8, scales, gamma, eps,
                     weight_offset, scale_ub, rows, cols, P, &a, out_format);
  if (st != ARNFP8_OK) return st;
  RowConfig cfg;  // after validation: the automatic choice queries the device
  st = resolve_row_config(opt, rows, (int)(cols / 8), P, &cfg);
  if (st != ARNFP8_OK) return st;
  return launch(row_table(out_format, P, cfg.vpt, residual_in != nullptr, residual_out != nullptr,
                          cfg.sc1_stores != 0),
                dim3(cfg.grid), dim3(cfg.threads), stream, a);
}

extern "C" int arnfp8_run_ex(const void *const *inputs, const void *residual_in,
                             void *residual_out, void *out_fp8, float *scales, const void *gamma,
                             float eps, float weight_offset, float scale_ub, int64_t rows,
                             int64_t cols, int P, hipStream_t stream, const arnfp8_launch *opt) {
  return arnfp8_run_fmt(inputs, residual_in, residual_out, out_fp8, scales, gamma, eps,
                        weight_offset, scale_ub, rows, cols, P, ARNFP8_FMT_E4M3FN, stream, opt);
}

extern "C" int arnfp8_run(const void *const *inputs, const void *residual_in, void *residual_out,
                          void *out_fp8, float *scales, const void *gamma, float eps,
                          float weight_offset, float scale_ub, int64_t rows, int64_t cols, int P,
                          hipStream_t stream) {
  return arnfp8_run_ex(inputs, residual_in, residual_out, out_fp8, scales, gamma, eps,
                       weight_offset, scale_ub, rows, cols, P, stream, nullptr);
}

extern "C" int64_t arnfp8_stage_bytes(int64_t rows, int64_t cols, int ngpus) {
  if (rows < 0 || cols <= 0 || ngpus < 1) return -1;
  const int64_t S = (rows + ngpus - 1) / ngpus;
  if (S > 0 && cols > (INT64_MAX / 2) / S) return -1;
  const int64_t scale_bytes = S * (int64_t)sizeof(float);
  return S * cols + (scale_bytes + ARNFP8_SIMD_WIDTH - 1) / ARNFP8_SIMD_WIDTH * ARNFP8_SIMD_WIDTH;
}

extern "C" int arnfp8_run_share(const void *const *inputs, const void *residual_in,
                                void *residual_out, void *staging, const void *gamma, float eps,
                                float weight_offset, float scale_ub, int64_t rows, int64_t cols,
                                int P, int ngpus, int rank, hipStream_t stream) {
  int st = check_shape(rows, cols, P);
  if (st != ARNFP8_OK) return st;
  if (ngpus < 1 || rank < 0 || rank >= ngpus) return ARNFP8_BAD_SHARE;
  st = check_scalars(eps, weight_offset, scale_ub, true);
  if (st != ARNFP8_OK) return st;
  if (rows == 0) return ARNFP8_OK;
  st = check_inputs(inputs, P);
  if (st != ARNFP8_OK) return st;
  if (staging == nullptr) return ARNFP8_NULL_POINTER;
  if (!aligned(staging, 16)) return ARNFP8_MISALIGNED;

  const int64_t S = (rows + ngpus - 1) / ngpus;
  const int64_t first = (int64_t)rank * S < rows ? (int64_t)rank * S : rows;
  const int64_t count = (first + S < rows ? first + S : rows) - first;
  // The share's rows of every full-size tensor (bf16: 2 bytes per element).
  const uintptr_t skip = (uintptr_t)(first * cols * 2);
  const void *shifted[ARNFP8_MAX_P];
  for (int p = 0; p < P; ++p) shifted[p] = (const char *)inputs[p] + skip;
  const void *rin = residual_in ? (const char *)residual_in + skip : nullptr;
  void *rout = residual_out ? (char *)residual_out + skip : nullptr;
  uint8_t *out = (uint8_t *)staging;
  float *scales = (float *)(out + S * cols);

  if (gamma == nullptr) return ARNFP8_NULL_POINTER;
  // The whole slot must stay clear of every full-size input and output.
  const Range slot{(uintptr_t)staging,
                   (uintptr_t)staging + (uintptr_t)arnfp8_stage_bytes(rows, cols, ngpus)};
  const uintptr_t full = (uintptr_t)(rows * cols * 2);
  for (int p = 0; p < P; ++p)
    if (overlaps(slot, Range{(uintptr_t)inputs[p], (uintptr_t)inputs[p] + full})) return ARNFP8_ALIAS;
  if (residual_in && overlaps(slot, Range{(uintptr_t)residual_in, (uintptr_t)residual_in + full}))
    return ARNFP8_ALIAS;
  if (residual_out && overlaps(slot, Range{(uintptr_t)residual_out, (uintptr_t)residual_out + full}))
    return ARNFP8_ALIAS;
  if (overlaps(slot, Range{(uintptr_t)gamma, (uintptr_t)gamma + 2 * (uintptr_t)cols}))
    return ARNFP8_ALIAS;
  if (count == 0) {
    if (!aligned(gamma, 16) || (residual_in && !aligned(residual_in, 16)) ||
        (residual_out && !aligned(residual_out, 16)))
      return ARNFP8_MISALIGNED;
    return ARNFP8_OK;
  }

  RowArgs a;
  st = prepare_fused(shifted, rin, rout, out, scales, gamma, eps, weight_offset, scale_ub, count,
                     cols, P, &a);
  if (st != ARNFP8_OK) return st;
  RowConfig cfg;
  st = resolve_row_config(nullptr, count, (int)(cols / 8), P, &cfg);
  if (st != ARNFP8_OK) return st;
  return launch(row_table(ARNFP8_FMT_E4M3FN, P, cfg.vpt, residual_in != nullptr,
                          residual_out != nullptr, cfg.sc1_stores != 0),
                dim3(cfg.grid), dim3(cfg.threads), stream, a);
}

extern "C" int64_t arnfp8_split_workspace_bytes(int64_t rows) {
  if (rows < 0 || rows > INT64_MAX / (16 * kSplitSlots)) return -1;
  return rows * 2 * kSplitSlots * (int64_t)sizeof(unsigned long long);
}

namespace {

// The largest power of two up to kSplitSlots that keeps the grid within one
// workgroup per CU and every part at least one full wave of chunks, and at
// least enough parts for 1024 lanes.  Measured on MI355X (graph replay,
// inputs out of cache): one row of 8192 columns, P = 8, in 8 parts 4.71
// against 5.89 us in one workgroup; 128 rows in 2 parts 7.40 against 7.77 us;
// 4 rows of 256 columns in 8 parts of 4 chunks 5.76 against 2.89 us (the
// exchange is then all overhead).
int auto_split_parts(int64_t rows, int c16) {
  const int64_t cus = device_cus();
  int parts = 1;
  while (parts * 2 <= kSplitSlots && rows * parts * 2 <= cus && c16 >= 64 * parts * 2) parts *= 2;
  while (c16 > 1024 * parts && parts < kSplitSlots) parts *= 2;
  return parts;
}

// A validated split call: the kernel, its arguments and its launch shape;
// with one part per row, the row kernel of arnfp8_run instead.
struct SplitCall {
  SplitKernel kernel;
  SplitArgs args;
  RowKernel row_kernel;
  RowArgs row_args;
  dim3 grid, block;
};

int launch_split(const SplitCall &c, hipStream_t stream) {
  if (c.row_kernel != nullptr) return launch(c.row_kernel, c.grid, c.block, stream, c.row_args);
  return launch(c.kernel, c.grid, c.block, stream, c.args);
}

// Validates a split call in the documented order and fills `call`.  Returns
// ARNFP8_OK with neither kernel set when there is nothing to launch (rows ==
// 0); the workspace is only looked at when there is.  With `own_workspace`
// the workspace is the library's array, set by the caller afterwards, and is
// not checked.
int prepare_split(const void *const *inputs, const void *residual_in, void *residual_out,
                  void *out_fp8, float *scales, const void *gamma, float eps, float weight_offset,
                  float scale_ub, int64_t rows, int64_t cols, int P, void *workspace,
                  int64_t workspace_bytes, const arnfp8_split_opts *opt, SplitCall *call,
                  bool own_workspace = false) {
  call->kernel = nullptr;
  call->row_kernel = nullptr;
  int st = check_shape(rows, cols, P);
  if (st != ARNFP8_OK) return st;
  st = check_scalars(eps, weight_offset, scale_ub, true);
  if (st != ARNFP8_OK) return st;
  const int c16 = (int)(cols / 8);
  int parts = opt ? opt->parts : 0;
  if (parts < 0 || parts > kSplitSlots) return ARNFP8_BAD_CONFIG;
  if (parts > 0 && c16 > 1024 * parts) return ARNFP8_BAD_CONFIG;
  if (rows == 0) return ARNFP8_OK;
  SplitArgs &a = call->args;
  {
    RowArgs &r = call->row_args;
    st = prepare_fused(inputs, residual_in, residual_out, out_fp8, scales, gamma, eps,
                       weight_offset, scale_ub, rows, cols, P, &r);
    if (st != ARNFP8_OK) return st;
    // A part may re-read a late partner's residual input, so it must stay
    // unmodified: no in-place update on this path.
    if (residual_in != nullptr && residual_in == residual_out) return ARNFP8_ALIAS;
    a.in = r.in;
    a.res_in = r.res_in;
    a.res_out = r.res_out;
    a.out = r.out;
    a.scales = r.scales;
    a.gamma = r.gamma;
    a.eps = r.eps;
    a.woff = r.woff;
    a.ub = r.ub;
    a.inv_cols = r.inv_cols;
    a.rows = r.rows;
    a.c16 = r.c16;
  }
  const int64_t need = arnfp8_split_workspace_bytes(rows);
  if (!own_workspace) {
    if (workspace == nullptr) return ARNFP8_NULL_POINTER;
    if (!aligned(workspace, 16)) return ARNFP8_MISALIGNED;
    if (need < 0 || workspace_bytes < need) return ARNFP8_BAD_WORKSPACE;
    const Range ws{(uintptr_t)workspace, (uintptr_t)workspace + (uintptr_t)need};
    const uintptr_t n = (uintptr_t)(rows * cols);
    for (int p = 0; p < P; ++p)
      if (overlaps(ws, Range{(uintptr_t)inputs[p], (uintptr_t)inputs[p] + 2 * n})) return ARNFP8_ALIAS;
    if (residual_in && overlaps(ws, Range{(uintptr_t)residual_in, (uintptr_t)residual_in + 2 * n}))
      return ARNFP8_ALIAS;
    if (residual_out && overlaps(ws, Range{(uintptr_t)residual_out, (uintptr_t)residual_out + 2 * n}))
      return ARNFP8_ALIAS;
    if (overlaps(ws, Range{(uintptr_t)out_fp8, (uintptr_t)out_fp8 + n}) ||
        overlaps(ws, Range{(uintptr_t)scales, (uintptr_t)scales + 4 * (uintptr_t)rows}) ||
        overlaps(ws, Range{(uintptr_t)gamma, (uintptr_t)gamma + 2 * (uintptr_t)cols}))
      return ARNFP8_ALIAS;
  }
  if (parts == 0) {
    parts = auto_split_parts(rows, c16);
    if (c16 > 1024 * parts) return ARNFP8_BAD_CONFIG;
  }
  if (parts == 1) {
    // Nothing to trade: arnfp8_run's kernel and launch shape, and the
    // workspace is left as it is (its per-row counts stay equal).
    const RowConfig cfg = pick_row_config(rows, c16, P);
    call->row_kernel = row_table(ARNFP8_FMT_E4M3FN, P, cfg.vpt, residual_in != nullptr,
                                 residual_out != nullptr, false);
    call->grid = dim3(cfg.grid);
    call->block = dim3(cfg.threads);
    return ARNFP8_OK;
  }
  if (rows * parts > (int64_t)INT32_MAX) return ARNFP8_BAD_SHAPE;
  a.ws = (unsigned long long *)workspace;
  a.parts = parts;
  a.cpp = (c16 + parts - 1) / parts;
  const int spin = opt ? opt->spin_polls : 0;
  a.spin_polls = spin == 0 ? 32768 : (spin < 0 ? -1 : spin);
  call->grid = dim3((unsigned)(rows * parts));
  call->block = dim3((a.cpp + 63) / 64 * 64);
  call->kernel = split_table(P, residual_in != nullptr, residual_out != nullptr);
  return ARNFP8_OK;
}

}  // namespace

extern "C" int arnfp8_split_parts(int64_t rows, int64_t cols) {
  if (check_shape(rows, cols, 1) != ARNFP8_OK || rows == 0) return -1;
  const int c16 = (int)(cols / 8);
  const int parts = auto_split_parts(rows, c16);
  return c16 > 1024 * parts ? -1 : parts;
}

extern "C" int arnfp8_run_split(const void *const *inputs, const void *residual_in,
                                void *residual_out, void *out_fp8, float *scales,
                                const void *gamma, float eps, float weight_offset, float scale_ub,
                                int64_t rows, int64_t cols, int P, void *workspace,
                                int64_t workspace_bytes, hipStream_t stream,
                                const arnfp8_split_opts *opt) {
  SplitCall c;
  const int st = prepare_split(inputs, residual_in, residual_out, out_fp8, scales, gamma, eps,
                               weight_offset, scale_ub, rows, cols, P, workspace,
                               workspace_bytes, opt, &c);
  if (st != ARNFP8_OK || (c.kernel == nullptr && c.row_kernel == nullptr)) return st;
  return launch_split(c, stream);
}

// ---- allocation-free split rows -------------------------------------------
//
// The workspace of arnfp8_run_split_noalloc is this device array: 128 bytes
// per row for up to ARNFP8_NOALLOC_MAX_ROWS rows (512 KiB), held by every
// device the library runs on until the process ends.  Host code never uses
// the array's name as an address: the address is looked up once per device
// (hipGetSymbolAddress, with that device current) and kept in scratch_ptr.

static __device__ __align__(256) unsigned long long
    scratch[ARNFP8_NOALLOC_MAX_ROWS * 2 * arnfp8::kSplitSlots];

namespace {

constexpr int kMaxDevices = 64;
constexpr int64_t kScratchWords = ARNFP8_NOALLOC_MAX_ROWS * 2 * arnfp8::kSplitSlots;

std::atomic<unsigned long long *> scratch_ptr[kMaxDevices];
std::atomic<bool> scratch_cleared[kMaxDevices];
std::mutex scratch_setup;

// Sets every word of the array to zero (a kernel, not a memset, so that it
// may also be recorded into a graph).
__global__ __launch_bounds__(256) void zero_words_kernel(unsigned long long *p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0ull;
}

// The current device's index and its copy of the array.
int scratch_for_current_device(int *dev, unsigned long long **ptr) {
  if (hipGetDevice(dev) != hipSuccess || *dev < 0 || *dev >= kMaxDevices) return ARNFP8_HIP_ERROR;
  unsigned long long *p = scratch_ptr[*dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(scratch_setup);
    p = scratch_ptr[*dev].load(std::memory_order_acquire);
    if (p == nullptr) {
      void *q = nullptr;
      if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr)
        return ARNFP8_HIP_ERROR;
      p = (unsigned long long *)q;
      scratch_ptr[*dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return ARNFP8_OK;
}

}  // namespace

extern "C" int arnfp8_run_split_noalloc(const void *const *inputs, const void *residual_in,
                                        void *residual_out, void *out_fp8, float *scales,
                                        const void *gamma, float eps, float weight_offset,
                                        float scale_ub, int64_t rows, int64_t cols, int P,
                                        hipStream_t stream, const arnfp8_split_opts *opt) {
  int st = check_shape(rows, cols, P);
  if (st != ARNFP8_OK) return st;
  if (rows > ARNFP8_NOALLOC_MAX_ROWS) return ARNFP8_BAD_WORKSPACE;
  // Every check first; the array is looked up only for a launch that uses it.
  SplitCall c;
  st = prepare_split(inputs, residual_in, residual_out, out_fp8, scales, gamma, eps,
                     weight_offset, scale_ub, rows, cols, P, nullptr, 0, opt, &c, true);
  if (st != ARNFP8_OK) return st;
  if (c.kernel == nullptr) {  // rows == 0, or one part per row (the row kernel)
    return c.row_kernel == nullptr ? ARNFP8_OK : launch_split(c, stream);
  }
  int dev = 0;
  unsigned long long *ws = nullptr;
  st = scratch_for_current_device(&dev, &ws);
  if (st != ARNFP8_OK) return st;
  c.args.ws = ws;
  if (!scratch_cleared[dev].load(std::memory_order_acquire)) {
    // The per-row counts must start equal: clear the whole array once, ahead
    // of the first launch on this device.  Under graph capture (or if the
    // capture state cannot be read) the clear is recorded with the call and
    // the device stays marked as not cleared, so the next call clears again.
    st = launch(zero_words_kernel, dim3(256), dim3(256), stream, ws, kScratchWords);
    if (st != ARNFP8_OK) return st;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusActive;
    if (hipStreamIsCapturing(stream, &cap) == hipSuccess && cap == hipStreamCaptureStatusNone)
      scratch_cleared[dev].store(true, std::memory_order_release);
  }
  return launch_split(c, stream);
}

extern "C" int arnfp8_convert_f32(const float *in, void *out, int64_t n, int format,
                                  hipStream_t stream) {
  if (format != ARNFP8_FMT_E4M3FN && format != ARNFP8_FMT_E5M2 && format != ARNFP8_CVT_BF16)
    return ARNFP8_BAD_FORMAT;
  if (n < 0 || n % 8 != 0 || n > INT64_MAX / 4) return ARNFP8_BAD_SHAPE;
  if (n == 0) return ARNFP8_OK;
  if (in == nullptr || out == nullptr) return ARNFP8_NULL_POINTER;
  if (!aligned(in, 16) || !aligned(out, 16)) return ARNFP8_MISALIGNED;
  const uintptr_t out_bytes = (uintptr_t)n * (format == ARNFP8_CVT_BF16 ? 2 : 1);
  if (overlaps(Range{(uintptr_t)in, (uintptr_t)in + 4 * (uintptr_t)n},
               Range{(uintptr_t)out, (uintptr_t)out + out_bytes}))
    return ARNFP8_ALIAS;
  const int64_t n8 = n / 8;
  int64_t blocks = (n8 + 255) / 256;
  if (blocks > (int64_t)device_cus() * 8) blocks = (int64_t)device_cus() * 8;
  const u32x4 *src = (const u32x4 *)in;
  const dim3 grid((unsigned)blocks), block(256);
  if (format == ARNFP8_FMT_E4M3FN)
    return launch(cvt_kernel<ARNFP8_FMT_E4M3FN>, grid, block, stream, src, out, n8);
  if (format == ARNFP8_FMT_E5M2)
    return launch(cvt_kernel<ARNFP8_FMT_E5M2>, grid, block, stream, src, out, n8);
  return launch(cvt_kernel<ARNFP8_CVT_BF16>, grid, block, stream, src, out, n8);
}

extern "C" const char *arnfp8_status_string(int status) {
  switch (status) {
    case ARNFP8_OK: return "ok";
    case ARNFP8_NULL_POINTER: return "a required pointer is NULL";
    case ARNFP8_MISALIGNED: return "a pointer is not aligned (16 bytes; 4 for scales)";
    case ARNFP8_BAD_SHAPE: return "bad shape (rows >= 0, 0 < cols <= 65536, cols % 8 == 0)";
    case ARNFP8_BAD_P: return "P must be in [1, 8]";
    case ARNFP8_ALIAS: return "an output overlaps an input or another output";
    case ARNFP8_HIP_ERROR: return "the kernel launch failed";
    case ARNFP8_BAD_CONFIG: return "invalid launch configuration";
    case ARNFP8_BAD_SHARE: return "bad share: ngpus must be >= 1 and 0 <= rank < ngpus";
    case ARNFP8_BAD_FORMAT: return "unknown output format";
    case ARNFP8_BAD_SCALAR:
      return "bad scalar: eps must be finite and >= 0, weight_offset finite, scale_ub > 0";
    case ARNFP8_BAD_WORKSPACE:
      return "workspace too small: fewer than arnfp8_split_workspace_bytes(rows) bytes, or more "
             "than ARNFP8_NOALLOC_MAX_ROWS rows for the allocation-free call";
    default: return "unknown status";
  }
}
