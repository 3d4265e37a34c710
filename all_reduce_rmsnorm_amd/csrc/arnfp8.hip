// arnfp8.hip -- gfx950 (CDNA4) kernels and the C ABI of the fused all-reduce
// epilogue: rank-order fp32 sum of P bf16 slabs rounded once to bf16, optional
// residual add and write-back, RMSNorm with gamma + weight_offset, and per-row
// dynamic fp8 e4m3fn quantisation, in one launch.
//
// Sources: Modular Mojo API docs "allreduce_rmsnorm_fp8" (function summary,
// Args); b12x PR #283 "PCIeTwoShotBF16" (PR description); TensorRT-LLM PR
// #19836 (Description, RESIDUAL_RMS_NORM); tt-metal rmsnorm_2d.py
// (add_unit_offset).
//
// Design (HBM-bound, not a contraction, so no MFMA):
//  * One workgroup owns a row at a time; a row is cut into 16-byte chunks of
//    8 bf16 and lane t of a T-lane workgroup owns chunks t, t + T, ...  Every
//    global access is a 16-byte vector per lane, so a wave moves 1 KiB per
//    load instruction, fully coalesced.
//  * For each chunk the P slab loads (and the residual load) are issued
//    together, then summed in fp32 in rank order and rounded once with the
//    gfx950 packed bf16 conversion (round to nearest even).
//  * The row stays in registers as packed bf16 between the statistics pass and
//    the quantisation pass: the only global traffic is the algorithmic one.
//  * (sum h^2, max |h g|) are reduced across the wave with butterfly lane
//    exchanges and across waves through LDS with a single barrier per row;
//    the LDS slot alternates with the row parity so consecutive rows of a
//    grid-stride loop need no second barrier.
//  * fp8 values come from the gfx950 packed fp32 -> OCP e4m3fn conversion,
//    after an explicit clamp to +-448, so the conversion never overflows.
//  * Every lane reaches every barrier; chunk guards only guard data accesses.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "arnfp8.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kE4m3Max = 448.0f;
constexpr float kScaleFloor = 1.0f / 229376.0f;  // 1 / (448 * 512)

struct Slabs {
  const u32x4 *p[ARNFP8_MAX_P];
};

// ---------------------------------------------------------------- helpers --

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 -> one word of two bf16 (lo in bits 0..15), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v = __builtin_convertvector((f32x2){lo, hi}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

// Eight fp32 (already clamped to +-448) -> eight e4m3fn bytes, element k in
// byte k, round to nearest even.
__device__ __forceinline__ u32x2 pack_e4m3(const float v[8]) {
  int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w0, true);
  int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], w1, true);
  return (u32x2){(uint32_t)w0, (uint32_t)w1};
}

// Streaming accesses: every slab, residual and output byte is touched once,
// so loads and stores are non-temporal (they do not displace gamma in cache).
__device__ __forceinline__ u32x4 load16(const u32x4 *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store16(u32x4 *p, u32x4 v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store8(u32x2 *p, u32x2 v) { __builtin_nontemporal_store(v, p); }

// Rank-order sum of one chunk: rank 0's value starts the fp32 accumulator,
// ranks 1..P-1 are added in order, and the total is rounded once to bf16.
template <int P>
__device__ __forceinline__ u32x4 rank_order_sum(const u32x4 (&x)[P]) {
  float acc[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    acc[2 * w] = bf16_lo(x[0][w]);
    acc[2 * w + 1] = bf16_hi(x[0][w]);
  }
#pragma unroll
  for (int p = 1; p < P; ++p) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc[2 * w] += bf16_lo(x[p][w]);
      acc[2 * w + 1] += bf16_hi(x[p][w]);
    }
  }
  u32x4 s;
#pragma unroll
  for (int w = 0; w < 4; ++w) s[w] = pack_bf16(acc[2 * w], acc[2 * w + 1]);
  return s;
}

// h = bf16(fp32(s) + fp32(r)), elementwise on a chunk.
__device__ __forceinline__ u32x4 add_bf16(u32x4 s, u32x4 r) {
  u32x4 h;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    h[w] = pack_bf16(bf16_lo(s[w]) + bf16_lo(r[w]), bf16_hi(s[w]) + bf16_hi(r[w]));
  return h;
}

// Butterfly reductions across the 64 lanes of a wave; every lane gets the result.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// ---------------------------------------------------------------- kernels --

// Sum only: a flat grid-stride stream over all 16-byte chunks of the tensor.
template <int P, int U>
__global__ __launch_bounds__(256) void arn_sum_kernel(Slabs in, u32x4 *__restrict__ out,
                                                      int64_t n16) {
  const int64_t T = blockDim.x;
  const int64_t stride = (int64_t)gridDim.x * T * U;
  for (int64_t base = (int64_t)blockIdx.x * T * U + threadIdx.x; base < n16; base += stride) {
    u32x4 x[U][P];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = base + u * T;
      if (c < n16) {
#pragma unroll
        for (int p = 0; p < P; ++p) x[u][p] = load16(in.p[p] + c);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = base + u * T;
      if (c < n16) store16(out + c, rank_order_sum<P>(x[u]));
    }
  }
}

struct RowArgs {
  Slabs in;
  const u32x4 *res_in;
  u32x4 *res_out;
  u32x2 *out;  // 8 fp8 per chunk
  float *scales;
  const u32x4 *gamma;
  float eps, woff, ub;
  float cols_f;
  int64_t rows;
  int c16;  // 16-byte chunks per row
};

// Loads in flight per lane in the statistics pass: chunks are processed in
// groups of G whose P slab loads (plus residual and gamma) are all issued
// before any of them is consumed.
// The budget is 24 loads (96 VGPRs), less what the fp32 h*g values of the
// row (8 VGPRs per chunk) leave free under ~200 VGPRs.
template <int P, int VPT, bool RES_IN>
constexpr int load_group() {
  const int budget = (200 - 8 * VPT) / 4 < 24 ? (200 - 8 * VPT) / 4 : 24;
  int g = 1;
  while (g * 2 <= VPT && g * 2 * (P + 1 + (RES_IN ? 1 : 0)) <= budget) g *= 2;
  return g;
}

// fl32(h * (g + weight_offset)) for the two bf16 elements of one word; the
// statistics and the quantisation pass both use exactly this expression.
__device__ __forceinline__ void gain2(uint32_t h, uint32_t g, float woff, float &lo, float &hi) {
  lo = bf16_lo(h) * (bf16_lo(g) + woff);
  hi = bf16_hi(h) * (bf16_hi(g) + woff);
}

// Fused epilogue: workgroups walk the rows grid-stride; lane t owns chunks
// t + v*T (v < VPT) of the row.  Between the statistics pass and the
// quantisation pass the row stays in registers: as fp32 h*g for up to 8
// chunks per lane, as packed bf16 h (gamma re-read from cache) for 16.
// Chunk indices past the end of a ragged row are clamped to the row's last
// chunk for the loads (an in-bounds duplicate read), and every store and
// statistic of such a chunk is masked.
template <int P, int VPT, bool RES_IN, bool RES_OUT>
__global__ __launch_bounds__(512) void arnfp8_row_kernel(RowArgs a) {
  constexpr int G = load_group<P, VPT, RES_IN>();
  constexpr bool KEEP_HG = VPT <= 8;
  __shared__ float red[2][8][2];  // [row parity][wave][sum h^2, max |h g|]
  const int t = threadIdx.x;
  const int T = blockDim.x;
  const int wave = t >> 6;
  const int nwaves = T >> 6;
  const int last = a.c16 - 1;
  int parity = 0;

  for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x, parity ^= 1) {
    // Row-uniform bases (scalar registers); lanes add a 32-bit chunk index.
    const int64_t base = row * (int64_t)a.c16;
    const u32x4 *xs[P];
#pragma unroll
    for (int p = 0; p < P; ++p) xs[p] = a.in.p[p] + base;
    const u32x4 *rin = RES_IN ? a.res_in + base : nullptr;
    u32x4 *rout = RES_OUT ? a.res_out + base : nullptr;
    u32x2 *qout = a.out + base;
    float hg[KEEP_HG ? VPT : 1][8];
    u32x4 hk[KEEP_HG ? 1 : VPT];
    float ss = 0.0f, mx = 0.0f;

#pragma unroll
    for (int v0 = 0; v0 < VPT; v0 += G) {
      u32x4 x[G][P], r[G], g[G];
#pragma unroll
      for (int k = 0; k < G; ++k) {
        const int c = min((v0 + k) * T + t, last);
#pragma unroll
        for (int p = 0; p < P; ++p) x[k][p] = load16(xs[p] + c);
        if constexpr (RES_IN) r[k] = load16(rin + c);
        g[k] = a.gamma[c];
      }
#pragma unroll
      for (int k = 0; k < G; ++k) {
        const int v = v0 + k;
        const bool valid = v * T + t <= last;
        u32x4 hv = rank_order_sum<P>(x[k]);
        if constexpr (RES_IN) hv = add_bf16(hv, r[k]);
        if constexpr (RES_OUT) {
          if (valid) store16(rout + v * T + t, hv);
        }
        if constexpr (!KEEP_HG) hk[v] = hv;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          float y0, y1;
          gain2(hv[w], g[k][w], a.woff, y0, y1);
          if constexpr (KEEP_HG) {
            hg[v][2 * w] = y0;
            hg[v][2 * w + 1] = y1;
          }
          if (valid) {
            const float h0 = bf16_lo(hv[w]), h1 = bf16_hi(hv[w]);
            ss += h0 * h0;
            ss += h1 * h1;
            mx = fmaxf(mx, fmaxf(fabsf(y0), fabsf(y1)));
          }
        }
      }
      // Keep the next group's loads below this point: hoisting them would
      // hold more loads in registers than the budget allows.
      if constexpr (G < VPT) __builtin_amdgcn_sched_barrier(0);
    }

    ss = wave_sum(ss);
    mx = wave_max(mx);
    if ((t & 63) == 0) {
      red[parity][wave][0] = ss;
      red[parity][wave][1] = mx;
    }
    __syncthreads();
    float tot = 0.0f, m = 0.0f;
    for (int w = 0; w < nwaves; ++w) {
      tot += red[parity][w][0];
      m = fmaxf(m, red[parity][w][1]);
    }

    const float r = 1.0f / sqrtf(tot / a.cols_f + a.eps);
    const float amax = m * r;
    const float scale = fmaxf(fminf(amax, a.ub) / kE4m3Max, kScaleFloor);
    const float cq = r / scale;
    if (t == 0) a.scales[row] = scale;

    constexpr int QG = KEEP_HG ? 1 : 4;  // gamma re-reads issued together
#pragma unroll
    for (int v0 = 0; v0 < VPT; v0 += QG) {
      u32x4 g[QG];
      if constexpr (!KEEP_HG) {
#pragma unroll
        for (int k = 0; k < QG; ++k) g[k] = a.gamma[min((v0 + k) * T + t, last)];
      }
      if constexpr (!KEEP_HG) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < QG; ++k) {
        const int v = v0 + k;
        const int c = v * T + t;
        float y[8];
        if constexpr (KEEP_HG) {
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] = hg[v][e];
        } else {
#pragma unroll
          for (int w = 0; w < 4; ++w) gain2(hk[v][w], g[k][w], a.woff, y[2 * w], y[2 * w + 1]);
        }
        if (c <= last) {
          float q[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) q[e] = fminf(fmaxf(y[e] * cq, -kE4m3Max), kE4m3Max);
          store8(qout + c, pack_e4m3(q));
        }
      }
    }
  }
}

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

int check_inputs(const void *const *inputs, int P) {
  if (inputs == nullptr) return ARNFP8_NULL_POINTER;
  for (int p = 0; p < P; ++p)
    if (inputs[p] == nullptr) return ARNFP8_NULL_POINTER;
  for (int p = 0; p < P; ++p)
    if (!aligned(inputs[p], 16)) return ARNFP8_MISALIGNED;
  return ARNFP8_OK;
}

int launch_status() {
  return hipGetLastError() == hipSuccess ? ARNFP8_OK : ARNFP8_HIP_ERROR;
}

int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// ---- launch tables: one entry per template instance ----

typedef void (*SumKernel)(Slabs, u32x4 *, int64_t);

template <int P>
SumKernel sum_kernel_for() {
  return arn_sum_kernel<P, 2>;
}

SumKernel sum_table(int P) {
  switch (P) {
    case 1: return sum_kernel_for<1>();
    case 2: return sum_kernel_for<2>();
    case 3: return sum_kernel_for<3>();
    case 4: return sum_kernel_for<4>();
    case 5: return sum_kernel_for<5>();
    case 6: return sum_kernel_for<6>();
    case 7: return sum_kernel_for<7>();
    default: return sum_kernel_for<8>();
  }
}

typedef void (*RowKernel)(RowArgs);

template <int P, int VPT>
RowKernel row_kernel_res(bool res_in, bool res_out) {
  if (res_in) return res_out ? arnfp8_row_kernel<P, VPT, true, true> : arnfp8_row_kernel<P, VPT, true, false>;
  return res_out ? arnfp8_row_kernel<P, VPT, false, true> : arnfp8_row_kernel<P, VPT, false, false>;
}

template <int P>
RowKernel row_kernel_vpt(int vpt, bool res_in, bool res_out) {
  switch (vpt) {
    case 1: return row_kernel_res<P, 1>(res_in, res_out);
    case 2: return row_kernel_res<P, 2>(res_in, res_out);
    case 4: return row_kernel_res<P, 4>(res_in, res_out);
    case 8: return row_kernel_res<P, 8>(res_in, res_out);
    default: return row_kernel_res<P, 16>(res_in, res_out);
  }
}

RowKernel row_table(int P, int vpt, bool res_in, bool res_out) {
  switch (P) {
    case 1: return row_kernel_vpt<1>(vpt, res_in, res_out);
    case 2: return row_kernel_vpt<2>(vpt, res_in, res_out);
    case 3: return row_kernel_vpt<3>(vpt, res_in, res_out);
    case 4: return row_kernel_vpt<4>(vpt, res_in, res_out);
    case 5: return row_kernel_vpt<5>(vpt, res_in, res_out);
    case 6: return row_kernel_vpt<6>(vpt, res_in, res_out);
    case 7: return row_kernel_vpt<7>(vpt, res_in, res_out);
    default: return row_kernel_vpt<8>(vpt, res_in, res_out);
  }
}

struct RowConfig {
  int threads;
  int vpt;
  int grid;
};

// Smallest chunks-per-lane (1, 2, 4, 8, 16) that fits the row in at most 512
// lanes; lanes rounded up to whole waves.
RowConfig pick_row_config(int64_t rows, int c16) {
  static const int vpts[5] = {1, 2, 4, 8, 16};
  RowConfig cfg{64, 16, 1};
  for (int i = 0; i < 5; ++i) {
    const int lanes = (c16 + vpts[i] - 1) / vpts[i];
    if (lanes <= 512) {
      cfg.vpt = vpts[i];
      cfg.threads = ((lanes + 63) / 64) * 64;
      break;
    }
  }
  cfg.grid = (int)(rows < 65536 ? rows : 65536);
  return cfg;
}

// Validates the fused call's arguments and fills the kernel arguments.
int prepare_fused(const void *const *inputs, const void *residual_in, void *residual_out,
                  void *out_fp8, float *scales, const void *gamma, float eps,
                  float weight_offset, float scale_ub, int64_t rows, int64_t cols, int P,
                  RowArgs *a) {
  int st = check_inputs(inputs, P);
  if (st != ARNFP8_OK) return st;
  if (out_fp8 == nullptr || scales == nullptr || gamma == nullptr) return ARNFP8_NULL_POINTER;
  if (!aligned(out_fp8, 16) || !aligned(gamma, 16) || !aligned(scales, 4) ||
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
  outs[nout++] = Range{(uintptr_t)scales, (uintptr_t)scales + 4 * (uintptr_t)rows};
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
  a->scales = scales;
  a->gamma = (const u32x4 *)gamma;
  a->eps = eps;
  a->woff = weight_offset;
  a->ub = scale_ub;
  a->cols_f = (float)cols;
  a->rows = rows;
  a->c16 = (int)(cols / 8);
  return ARNFP8_OK;
}

// Resolves the launch options against the automatic choice.
int resolve_row_config(const arnfp8_launch *opt, int64_t rows, int c16, RowConfig *cfg) {
  *cfg = pick_row_config(rows, c16);
  if (opt == nullptr) return ARNFP8_OK;
  if (opt->variant != ARNFP8_VARIANT_AUTO && opt->variant != ARNFP8_VARIANT_ROW)
    return ARNFP8_BAD_CONFIG;
  if (opt->threads < 0 || opt->vpt < 0 || opt->grid < 0) return ARNFP8_BAD_CONFIG;
  if (opt->threads) {
    if (opt->threads % 64 != 0 || opt->threads > 512) return ARNFP8_BAD_CONFIG;
    cfg->threads = opt->threads;
    if (!opt->vpt) {  // the smallest chunks-per-lane that covers the row
      static const int vpts[5] = {1, 2, 4, 8, 16};
      cfg->vpt = 0;
      for (int i = 0; i < 5 && !cfg->vpt; ++i)
        if ((int64_t)vpts[i] * cfg->threads >= c16) cfg->vpt = vpts[i];
      if (!cfg->vpt) return ARNFP8_BAD_CONFIG;
    }
  }
  if (opt->vpt) {
    if (opt->vpt != 1 && opt->vpt != 2 && opt->vpt != 4 && opt->vpt != 8 && opt->vpt != 16)
      return ARNFP8_BAD_CONFIG;
    cfg->vpt = opt->vpt;
    if (!opt->threads) cfg->threads = ((c16 + cfg->vpt - 1) / cfg->vpt + 63) / 64 * 64;
    if (cfg->threads > 512) return ARNFP8_BAD_CONFIG;
  }
  if ((int64_t)cfg->threads * cfg->vpt < c16) return ARNFP8_BAD_CONFIG;
  if (opt->grid) cfg->grid = opt->grid;
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
  const int threads = 256;
  const int U = 2;
  int64_t blocks = (n16 + threads * U - 1) / (threads * U);
  const int64_t cap = (int64_t)device_cus() * 16;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(sum_table(P), dim3((unsigned)blocks), dim3(threads), 0, stream, s, (u32x4 *)out,
                     n16);
  return launch_status();
}

extern "C" int arnfp8_run_ex(const void *const *inputs, const void *residual_in,
                             void *residual_out, void *out_fp8, float *scales, const void *gamma,
                             float eps, float weight_offset, float scale_ub, int64_t rows,
                             int64_t cols, int P, hipStream_t stream, const arnfp8_launch *opt) {
  int st = check_shape(rows, cols, P);
  if (st != ARNFP8_OK) return st;
  RowConfig cfg;
  st = resolve_row_config(opt, rows, (int)(cols / 8), &cfg);
  if (st != ARNFP8_OK) return st;
  if (rows == 0) return ARNFP8_OK;
  RowArgs a;
  st = prepare_fused(inputs, residual_in, residual_out, out_fp8, scales, gamma, eps,
                     weight_offset, scale_ub, rows, cols, P, &a);
  if (st != ARNFP8_OK) return st;
  hipLaunchKernelGGL(row_table(P, cfg.vpt, residual_in != nullptr, residual_out != nullptr),
                     dim3(cfg.grid), dim3(cfg.threads), 0, stream, a);
  return launch_status();
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

  RowConfig cfg;
  st = resolve_row_config(nullptr, count, (int)(cols / 8), &cfg);
  if (st != ARNFP8_OK) return st;
  RowArgs a;
  st = prepare_fused(shifted, rin, rout, out, scales, gamma, eps, weight_offset, scale_ub, count,
                     cols, P, &a);
  if (st != ARNFP8_OK) return st;
  hipLaunchKernelGGL(row_table(P, cfg.vpt, residual_in != nullptr, residual_out != nullptr),
                     dim3(cfg.grid), dim3(cfg.threads), 0, stream, a);
  return launch_status();
}

extern "C" const char *arnfp8_status_string(int status) {
  switch (status) {
    case ARNFP8_OK: return "ok";
    case ARNFP8_NULL_POINTER: return "a required pointer is NULL";
    case ARNFP8_MISALIGNED: return "a pointer is not aligned (16 bytes; 4 for scales)";
    case ARNFP8_BAD_SHAPE: return "bad shape (rows >= 0, 0 < cols <= 65536, cols % 8 == 0)";
    case ARNFP8_BAD_P: return "P must be in [1, 8]";
    case ARNFP8_ALIAS: return "an output overlaps an input or another output";
    case ARNFP8_HIP_ERROR: return "HIP launch error";
    case ARNFP8_BAD_CONFIG: return "invalid launch configuration";
    case ARNFP8_BAD_SHARE: return "bad share: ngpus must be >= 1 and 0 <= rank < ngpus";
    default: return "unknown status";
  }
}
