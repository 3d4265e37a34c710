// arnfp8_kernels.hpp -- gfx950 (CDNA4) device code of the fused all-reduce
// epilogue: the rank-order sum kernel, the fused row kernel and the
// conversion kernel.  Included by the C ABI (arnfp8.hip) and by the
// per-format instance units (arnfp8_rows_*.hip).
//
// Sources: Modular Mojo API docs "allreduce_rmsnorm_fp8" (function summary,
// Args); b12x PR #283 "PCIeTwoShotBF16" (PR description); TensorRT-LLM PR
// #19836 (Description, RESIDUAL_RMS_NORM); tt-metal rmsnorm_2d.py
// (add_unit_offset); Huawei CANN aclnnAlltoAllQuantMatmul (E5M2 and mx
// quantisation).
//
// Design (the path is HBM-bound and not a contraction, so no MFMA):
//  * A workgroup owns a row at a time (rows walked grid-stride).  A row is cut
//    into 16-byte chunks of 8 bf16; lane t of a T-lane workgroup owns chunks
//    t, t + T, ...  Every global access is a 16-byte vector per lane, so a
//    wave moves 1 KiB per instruction, fully coalesced.
//  * All P slab loads, the residual load and the gamma load of a lane's chunks
//    are issued before any is consumed (within a register budget); indices
//    past a ragged row's end are clamped for the loads and masked for stores
//    and statistics.  Slabs and residual are loaded non-temporally; the row
//    outputs are buffer stores whose cache policy the launch chooses.
//  * The sum is accumulated in fp32 in rank order and rounded once with the
//    packed bf16 conversion (round to nearest even); the residual add is
//    rounded the same way.
//  * fl32(h * g) stays in registers between the statistics pass and the
//    quantisation pass: the only global traffic is the algorithmic one.
//  * (sum h^2, max |h g|) are reduced across the wave with DPP moves inside
//    each row of 16 lanes and two lane-swap moves across rows, then across
//    waves through LDS with one barrier per row; the LDS slot alternates with
//    the row parity so consecutive rows need no second barrier.
//  * fp8 values come from the packed OCP e4m3fn / e5m2 conversions after an
//    explicit clamp, so a conversion never overflows.
//  * Every lane reaches every barrier and every lane exchange; guards only
//    guard data accesses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "arnfp8.h"

namespace arnfp8 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Output formats of the fused kernel.
constexpr int kFmtE4m3 = ARNFP8_FMT_E4M3FN;  // per-row fp32 scale, OCP e4m3fn
constexpr int kFmtE5m2 = ARNFP8_FMT_E5M2;    // per-row fp32 scale, OCP e5m2
constexpr int kFmtMx = ARNFP8_FMT_MXFP8;     // e4m3fn + one E8M0 scale per 32 values

// Largest finite value of the per-row formats; the row scale is floored at
// 1 / (fmax * 512).
template <int FMT>
constexpr float fmt_max() { return FMT == kFmtE5m2 ? 57344.0f : 448.0f; }
template <int FMT>
constexpr float fmt_floor() { return 1.0f / (fmt_max<FMT>() * 512.0f); }

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

// The same for OCP e5m2 (the gfx950 "bf8" conversion), values clamped to
// +-57344.
__device__ __forceinline__ u32x2 pack_e5m2(const float v[8]) {
  int w0 = __builtin_amdgcn_cvt_pk_bf8_f32(v[0], v[1], 0, false);
  w0 = __builtin_amdgcn_cvt_pk_bf8_f32(v[2], v[3], w0, true);
  int w1 = __builtin_amdgcn_cvt_pk_bf8_f32(v[4], v[5], 0, false);
  w1 = __builtin_amdgcn_cvt_pk_bf8_f32(v[6], v[7], w1, true);
  return (u32x2){(uint32_t)w0, (uint32_t)w1};
}

// MX shared exponent of a block whose largest magnitude is `amax` (fp32):
// floor(log2(amax)) - 8 (8 = exponent of the largest e4m3fn normal, 448),
// clamped to the E8M0 range [-127, 127]; an all-zero block takes -127.
__device__ __forceinline__ int mx_shared_exp(float amax) {
  if (amax == 0.0f) return -127;
  int e = __builtin_amdgcn_frexp_expf(amax) - 1 - 8;  // amax = m * 2^k, m in [0.5, 1)
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Streaming accesses: every slab, residual and output byte is touched once,
// so loads are non-temporal (they do not displace gamma in cache).
__device__ __forceinline__ u32x4 load16(const u32x4 *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store16(u32x4 *p, u32x4 v) { __builtin_nontemporal_store(v, p); }

// Row outputs go through buffer stores so that the cache policy can be chosen
// per launch: non-temporal (nt, the default) or sc1 (device-scope coherence).
// Measured on MI355X with a fresh set of output buffers on every call (the
// usual case: the outputs do not stay in the 256 MB Infinity Cache between
// calls), nt stores are the fastest policy: 8192 x 7168, P = 8 takes ~205 us
// with nt, ~211 us with sc1 and ~212 us with the default policy.  sc1 wins
// (~197 us) only when the same output buffers are rewritten while they are
// still cache-resident.  For decode batches nt is also the fastest (P = 4
// [32, 7168], inputs not in cache: 4.9 us nt, 5.2 us default policy).
// s_waitcnt operand (gfx9 encoding) that waits for vmcnt == 0 only: expcnt
// and lgkmcnt at their maxima (7 in bits 6:4, 15 in bits 11:8), vmcnt 0.
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr int kStoreNt = 2;    // cache-policy operand bit of nt
constexpr int kStoreSc1 = 16;  // cache-policy operand bit of sc1
// Word 3 of a raw (untyped, unswizzled, stride-0) buffer resource on
// gfx9-family targets: the 32-bit data format.
constexpr int kRawBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, kRawBufferWord3);
}
// The policy is a compile-time choice: a run-time branch around the stores
// splits the chunk loop and stops the compiler from issuing every slab load
// up front (measured: the gain is lost).
template <bool SC1>
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, int byte_off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, SC1 ? kStoreSc1 : kStoreNt);
}
template <bool SC1>
__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, int byte_off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, byte_off, 0, SC1 ? kStoreSc1 : kStoreNt);
}
template <bool SC1>
__device__ __forceinline__ void buf_store1(__amdgpu_buffer_rsrc_t r, int byte_off, uint8_t v) {
  __builtin_amdgcn_raw_buffer_store_b8(v, r, byte_off, 0, SC1 ? kStoreSc1 : kStoreNt);
}

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

// DPP lane exchanges inside a row of 16 lanes (VALU moves, no LDS): the
// partner lane is lane ^ 1 (quad_perm [1,0,3,2]), lane ^ 2 (quad_perm
// [2,3,0,1]), the mirror within 8 lanes, or the mirror within 16 lanes.
constexpr int kDppQuadXor1 = 0xB1;
constexpr int kDppQuadXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

// A lane whose partner is inactive reads 0 (bound_ctrl): the identity of
// every reduction below, whose operands are sums of squares and magnitudes.
// An identity there lets the compiler fold the move into the consuming
// add or max (one DPP instruction instead of a copy, a move and the op).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __uint_as_float(dpp_u<CTRL>(__float_as_uint(v)));
}

// The larger of two non-negative finite floats, compared as their bit
// patterns (for such values the unsigned order of the patterns is the order
// of the values): an integer max, which needs none of the NaN-quieting moves
// the compiler puts ahead of a float max whose operands it cannot prove
// canonical (values read from LDS or moved across lanes).
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ float max_nonneg(float a, float b) {
  return __uint_as_float(umax(__float_as_uint(a), __float_as_uint(b)));
}

// Pairs across rows with gfx950's lane-swap moves (VALU, no LDS round trip).
// Given the same value twice, v_permlane16_swap returns, at every lane, the
// values of lanes l and l ^ 16 (one in each result), and v_permlane32_swap
// those of lanes l and l ^ 32.  Both partners combine the same two values
// (the operations below commute), so they agree bit for bit.
__device__ __forceinline__ f32x2 pair16(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto s = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  // Elements are read into scalars first: a bit cast of a vector element
  // expression would read element 0 whatever the index.
  const uint32_t a = s[0], b = s[1];
  return (f32x2){__uint_as_float(a), __uint_as_float(b)};
}
__device__ __forceinline__ f32x2 pair32(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const uint32_t a = s[0], b = s[1];
  return (f32x2){__uint_as_float(a), __uint_as_float(b)};
}

// Reductions across the 64 lanes of a wave; every lane gets the result.
// Within a row of 16 lanes: xor 1, xor 2 (the quad), then the 8-lane and
// 16-lane mirrors, which pair each lane with one in the other half; across
// rows: the pairs at distance 16, then 32.  The order of the additions is
// fixed, so the sum is deterministic.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<kDppQuadXor1>(v);
  v += dpp<kDppQuadXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppMirror>(v);
  f32x2 p = pair16(v);
  v = p.x + p.y;
  p = pair32(v);
  return p.x + p.y;
}
// The maximum of non-negative finite values (magnitudes), on their bit
// patterns.
__device__ __forceinline__ float wave_max(float v) {
  uint32_t u = __float_as_uint(v);
  u = umax(u, dpp_u<kDppQuadXor1>(u));
  u = umax(u, dpp_u<kDppQuadXor2>(u));
  u = umax(u, dpp_u<kDppHalfMirror>(u));
  u = umax(u, dpp_u<kDppMirror>(u));
  f32x2 p = pair16(__uint_as_float(u));
  u = umax(__float_as_uint(p.x), __float_as_uint(p.y));
  p = pair32(__uint_as_float(u));
  return __uint_as_float(umax(__float_as_uint(p.x), __float_as_uint(p.y)));
}

// ---------------------------------------------------------------- kernels --

// Sum only: a flat grid-stride stream over all 16-byte chunks of the tensor,
// U chunks per lane per iteration.  With U == 4 (large tensors) the result is
// stored with nt buffer stores through a resource over the iteration's
// window; otherwise with plain nt stores.
template <int P, int U>
__global__ __launch_bounds__(256) void arn_sum_kernel(Slabs in, u32x4 *__restrict__ out,
                                                      int64_t n16) {
  const int64_t T = blockDim.x;
  const int64_t stride = (int64_t)gridDim.x * T * U;
  if constexpr (U == 4) {
    for (int64_t blk = (int64_t)blockIdx.x * T * U; blk < n16; blk += stride) {
      const int64_t base = blk + threadIdx.x;
      u32x4 x[U][P];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c = base + u * T;
        if (c < n16) {
#pragma unroll
          for (int p = 0; p < P; ++p) x[u][p] = load16(in.p[p] + c);
        }
      }
      // The window [blk, blk + T * U) clipped to the tensor; stores past its
      // end are dropped by the buffer range check as well as by the guard.
      const int64_t left = n16 - blk;
      const __amdgpu_buffer_rsrc_t w =
          row_rsrc(out + blk, (int)((left < T * U ? left : T * U) * 16));
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c = base + u * T;
        if (c < n16)
          buf_store16<false>(w, (int)((threadIdx.x + u * T) * 16), rank_order_sum<P>(x[u]));
      }
    }
  } else {
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
}

// The kernels' conversion steps on their own: 8 fp32 per lane per step ->
// e4m3fn (clamped to +-448), e5m2 (clamped to +-57344) or bf16 (round to
// nearest even, unclamped), exactly as the fused kernel converts.
template <int FMT>
__global__ __launch_bounds__(256) void cvt_kernel(const u32x4 *__restrict__ in,
                                                  void *__restrict__ out, int64_t n8) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride) {
    const u32x4 a = in[2 * i], b = in[2 * i + 1];
    float v[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[k] = __uint_as_float(a[k]);
      v[4 + k] = __uint_as_float(b[k]);
    }
    if constexpr (FMT == ARNFP8_CVT_BF16) {
      u32x4 w;
#pragma unroll
      for (int k = 0; k < 4; ++k) w[k] = pack_bf16(v[2 * k], v[2 * k + 1]);
      ((u32x4 *)out)[i] = w;
    } else {
      constexpr float lim = FMT == ARNFP8_FMT_E5M2 ? 57344.0f : 448.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = fminf(fmaxf(v[k], -lim), lim);
      ((u32x2 *)out)[i] = FMT == ARNFP8_FMT_E5M2 ? pack_e5m2(v) : pack_e4m3(v);
    }
  }
}

struct RowArgs {
  Slabs in;
  const u32x4 *res_in;
  u32x4 *res_out;
  u32x2 *out;  // 8 fp8 per chunk
  float *scales;       // per-row formats: fp32 [rows]
  uint8_t *mx_scales;  // MXFP8: E8M0 [rows, c16 / 4]
  const u32x4 *gamma;
  float eps, woff, ub;
  float inv_cols;  // fl32(1 / cols)
  int64_t rows;
  int c16;  // 16-byte chunks per row
};

// Arguments of the split-row kernel (arnfp8_split.hip): the row kernel's, plus
// the exchange workspace ([rows][kSplitSlots][2] 64-bit words), the parts per
// row, the chunks per part and the bound of the wait for a partner's words.
constexpr int kSplitSlots = 8;  // most parts a row can be split into
struct SplitArgs {
  Slabs in;
  const u32x4 *res_in;
  u32x4 *res_out;
  u32x2 *out;
  float *scales;
  const u32x4 *gamma;
  unsigned long long *ws;
  float eps, woff, ub;
  float inv_cols;
  int64_t rows;
  int c16;
  int parts;       // workgroups per row, 1..kSplitSlots
  int cpp;         // chunks per part, ceil(c16 / parts)
  int spin_polls;  // polls of a partner's words before computing its pair here
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
template <int FMT, int P, int VPT, bool RES_IN, bool RES_OUT, bool SC1>
__global__ __launch_bounds__(VPT == 1 ? 1024 : 512) void arnfp8_row_kernel(RowArgs a) {
  constexpr int G = load_group<P, VPT, RES_IN>();
  constexpr bool KEEP_HG = VPT <= 8;
  constexpr bool DEFER_STORES = P <= 4;  // residual stores after the group's loads
  __shared__ float red[2][16][2];  // [row parity][wave][sum h^2, max |h g|]
  const int t = threadIdx.x;
  const int T = blockDim.x;
  const int wave = t >> 6;
  const int nwaves = T >> 6;
  const int last = a.c16 - 1;
  int parity = 0;

  for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x, parity ^= 1) {
    // Wave priority: low while the row's loads are issued, high once they are
    // in flight (the reduction, quantisation and stores).  Measured on MI355X:
    // decode (P = 4, 32 x 7168) 3.62 against 3.68 us per call; prefill
    // unchanged; the opposite order costs prefill 1 %.
    __builtin_amdgcn_s_setprio(0);
    // Row-uniform bases (scalar registers); lanes add a 32-bit chunk index.
    const int64_t base = row * (int64_t)a.c16;
    const u32x4 *xs[P];
#pragma unroll
    for (int p = 0; p < P; ++p) xs[p] = a.in.p[p] + base;
    const u32x4 *rin = RES_IN ? a.res_in + base : nullptr;
    // Row outputs: buffer resources covering exactly this row's bytes.
    const __amdgpu_buffer_rsrc_t rout =
        row_rsrc(RES_OUT ? (const void *)(a.res_out + base) : (const void *)a.gamma,
                 RES_OUT ? a.c16 * 16 : 0);
    const __amdgpu_buffer_rsrc_t qout = row_rsrc(a.out + base, a.c16 * 8);
    const __amdgpu_buffer_rsrc_t mxout =
        FMT == kFmtMx ? row_rsrc(a.mx_scales + row * (int64_t)(a.c16 >> 2), a.c16 >> 2) : qout;
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
      if (v0 == 0) __builtin_amdgcn_s_setprio(3);
      u32x4 hs[G];
#pragma unroll
      for (int k = 0; k < G; ++k) {
        const int v = v0 + k;
        const bool valid = v * T + t <= last;
        u32x4 hv = rank_order_sum<P>(x[k]);
        if constexpr (RES_IN) hv = add_bf16(hv, r[k]);
        if constexpr (RES_OUT && !DEFER_STORES) {
          if (valid) buf_store16<SC1>(rout, (v * T + t) * 16, hv);
        }
        hs[k] = hv;
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
      // With up to four slabs (DEFER_STORES) the group's residual stores go
      // out only once every load of the group has arrived.  A store issued while loads are
      // still pending leaves reads and writes mixed in the one vector-memory
      // counter, and a later wait for a load (the gamma loads come last) then
      // waits for the store as well, which puts the store's completion on the
      // row's critical path ahead of the reduction.  The explicit wait is for
      // loads only (no store is pending yet).  Measured on MI355X, 512 x 2
      // lanes, inputs out of cache: P = 4 over 7168 columns 4.97 against
      // 5.11 us at 1 row, 5.47 / 5.58 at 32, 6.2 / 6.4 at 128, level from 512
      // rows; with eight slabs the early store is better (P = 8: 5.92 against
      // 6.03 us at 1 row; 205.3 against 206.7 us at 8192 rows), as waiting
      // for twenty loads delays the first store more than the late wait costs.
      if constexpr (RES_OUT && DEFER_STORES) {
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
#pragma unroll
        for (int k = 0; k < G; ++k) {
          const int v = v0 + k;
          if (v * T + t <= last) buf_store16<SC1>(rout, (v * T + t) * 16, hs[k]);
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
      m = max_nonneg(m, red[parity][w][1]);
    }

    // The row scalars sit on every row's critical path, so r and 1/scale use
    // the hardware reciprocal square root and reciprocal (each within 1 ulp;
    // measured: decode 3.49 against 3.61 us per call with the IEEE square root
    // and divisions).  The division by the format maximum stays IEEE, so a
    // clamped scale is exactly fl32(scale_ub / fmax).
    // eps = 0 on an all-zero row leaves nothing to normalise: r = 0 makes the
    // row all zeros (floor scale, zero codes) instead of 0 * inf = NaN.
    const float den = tot * a.inv_cols + a.eps;
    const float r = den > 0.0f ? __builtin_amdgcn_rsqf(den) : 0.0f;
    float cq = 0.0f;
    if constexpr (FMT != kFmtMx) {
      const float amax = m * r;
      const float scale = fmaxf(fminf(amax, a.ub) / fmt_max<FMT>(), fmt_floor<FMT>());
      cq = r * __builtin_amdgcn_rcpf(scale);
      if (t == 0) a.scales[row] = scale;
    }

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
        float q[8];
        if constexpr (FMT == kFmtMx) {
          // Block of 32 = the 4 consecutive chunks of lanes 4j..4j+3 (T is a
          // multiple of 64 and c16 of 4, so a quad is wholly valid or not).
          float bmax = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            y[e] = y[e] * r;
            bmax = fmaxf(bmax, fabsf(y[e]));
          }
          bmax = max_nonneg(bmax, dpp<kDppQuadXor1>(bmax));
          bmax = max_nonneg(bmax, dpp<kDppQuadXor2>(bmax));
          const int ex = mx_shared_exp(bmax);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            q[e] = fminf(fmaxf(__builtin_amdgcn_ldexpf(y[e], -ex), -448.0f), 448.0f);
          if (c <= last && (t & 3) == 0) buf_store1<SC1>(mxout, c >> 2, (uint8_t)(ex + 127));
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            q[e] = fminf(fmaxf(y[e] * cq, -fmt_max<FMT>()), fmt_max<FMT>());
        }
        if (c <= last) {
          buf_store8<SC1>(qout, c * 8, FMT == kFmtE5m2 ? pack_e5m2(q) : pack_e4m3(q));
        }
      }
    }
  }
}

}  // namespace arnfp8
