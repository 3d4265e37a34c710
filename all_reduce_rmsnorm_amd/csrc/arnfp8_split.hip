// arnfp8_split.hip -- the fused epilogue with each row split across several
// workgroups (the small-batch and one-token path of arnfp8_run_split).
//
// Sources: TensorRT-LLM PR #19836 (Description: at one token the
// RESIDUAL_RMS_NORM epilogue spreads a row over a cluster of 8 CTAs, which
// trade their partial sums); Modular Mojo API docs "allreduce_rmsnorm_fp8"
// (function summary, Args: the operation itself).
//
// CDNA4 has no clusters and no distributed shared memory, so the parts of a
// row trade their statistics through device memory:
//  * A row of c16 16-byte chunks is cut into `parts` consecutive ranges of
//    cpp = ceil(c16 / parts) chunks; workgroup b owns part b % parts of row
//    b / parts, one chunk per lane.  Loads, the rank-order sum, the residual
//    add and write-back, and fl32(h * g) are those of the row kernel.
//  * Each part reduces (sum h^2, max |h g|) over its chunks (DPP and lane
//    swaps in the wave, LDS across waves) and publishes the pair as two
//    64-bit words, each holding the value in its low half and a count in its
//    high half, with relaxed device-scope atomic stores: a word carries its
//    own validity, so no fence orders it against anything else.
//  * Lane j of the first wave then polls part j's words (all partners at
//    once) until both carry this launch's count.  The row's statistics are
//    the parts' pairs combined in part order, the same sum in every part, so
//    every part derives the same r, scale and 1/scale.
//  * Counts: the workspace holds kSplitSlots slots of two words per row.
//    Each launch raises every slot of each of its rows by one (part s writes
//    slot s, part 0 also the slots past the last part), so the slots of a
//    row always agree, whatever the shapes of earlier launches; a part reads
//    its own slot's count before publishing to learn this launch's count.
//    No host-side epoch is needed, and graph replays stay in step.  (A call
//    with one part per row launches the row kernel instead and leaves the
//    counts as they are.)
//  * The wait is bounded.  A part whose partner has not published when the
//    bound runs out computes that partner's pair itself, from the inputs,
//    with the partner's own lanes, chunk order and reductions, so the pair is
//    bitwise the one the partner publishes and the result does not depend on
//    which path ran.  This re-reads the partner's residual input, which is
//    why the residual cannot be updated in place on this path.
#include "arnfp8_tables.hpp"

namespace arnfp8 {

namespace {

// One chunk's loads: the P slabs, the residual and gamma.
template <int P, bool RES_IN>
struct ChunkIn {
  u32x4 x[P], r, g;
};

template <int P, bool RES_IN>
__device__ __forceinline__ void split_load(const SplitArgs &a, int64_t base, int c,
                                           ChunkIn<P, RES_IN> &in) {
#pragma unroll
  for (int p = 0; p < P; ++p) in.x[p] = load16(a.in.p[p] + base + c);
  if constexpr (RES_IN) in.r = load16(a.res_in + base + c);
  in.g = a.gamma[c];
}

// Forms h and fl32(h * g) from one chunk's loads, and adds the chunk's share
// of the statistics when `valid`.
template <int P, bool RES_IN>
__device__ __forceinline__ void split_chunk(const SplitArgs &a, const ChunkIn<P, RES_IN> &in,
                                            bool valid, u32x4 &hv, float hg[8], float &ss,
                                            float &mx) {
  hv = rank_order_sum<P>(in.x);
  if constexpr (RES_IN) hv = add_bf16(hv, in.r);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    gain2(hv[w], in.g[w], a.woff, hg[2 * w], hg[2 * w + 1]);
    if (valid) {
      const float h0 = bf16_lo(hv[w]), h1 = bf16_hi(hv[w]);
      ss += h0 * h0;
      ss += h1 * h1;
      mx = fmaxf(mx, fmaxf(fabsf(hg[2 * w]), fabsf(hg[2 * w + 1])));
    }
  }
}

// (sum, max) of the lanes' pairs over the workgroup, in a fixed order (the
// wave reductions, then the waves in order); LDS slot `slot` alternates
// between consecutive calls so that one barrier per call suffices.
__device__ __forceinline__ void block_pair(float ss, float mx, float (*red)[16][2], int slot,
                                           int wave, int nwaves, float &tot, float &m) {
  ss = wave_sum(ss);
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) {
    red[slot][wave][0] = ss;
    red[slot][wave][1] = mx;
  }
  __syncthreads();
  tot = 0.0f;
  m = 0.0f;
  for (int w = 0; w < nwaves; ++w) {
    tot += red[slot][w][0];
    m = max_nonneg(m, red[slot][w][1]);
  }
}

__device__ __forceinline__ unsigned long long ws_word(unsigned count, float v) {
  return ((unsigned long long)count << 32) | __float_as_uint(v);
}
__device__ __forceinline__ unsigned ws_count(unsigned long long w) { return (unsigned)(w >> 32); }
__device__ __forceinline__ float ws_value(unsigned long long w) {
  return __uint_as_float((unsigned)w);
}

}  // namespace

template <int P, bool RES_IN, bool RES_OUT>
__global__ __launch_bounds__(1024) void arnfp8_split_kernel(SplitArgs a) {
  __shared__ float red[2][16][2];
  __shared__ float part_ss[kSplitSlots], part_mx[kSplitSlots];
  __shared__ int missing[kSplitSlots];
  const int t = threadIdx.x;
  const int wave = t >> 6, nwaves = blockDim.x >> 6;
  const int64_t row = blockIdx.x / a.parts;
  const int part = blockIdx.x % a.parts;
  const int64_t base = row * (int64_t)a.c16;
  const int last = a.c16 - 1;
  unsigned long long *slots = a.ws + row * (2 * kSplitSlots);

  // This launch's count: one more than this part's slot holds (only this
  // workgroup writes that slot in this launch, and only after this read).
  const unsigned count =
      ws_count(__hip_atomic_load(slots + 2 * part, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) +
      1u;

  __builtin_amdgcn_s_setprio(0);
  const int first = part * a.cpp;
  const bool valid = t < a.cpp && first + t <= last;
  const int c = min(first + t, last);
  ChunkIn<P, RES_IN> in;
  split_load<P, RES_IN>(a, base, c, in);
  // Every load is issued before any is consumed (s_setprio orders the
  // scheduler as well as the wave).
  __builtin_amdgcn_s_setprio(3);
  u32x4 hv;
  float hg[8];
  float ss = 0.0f, mx = 0.0f;
  split_chunk<P, RES_IN>(a, in, valid, hv, hg, ss, mx);
  const __amdgpu_buffer_rsrc_t rout =
      row_rsrc(RES_OUT ? (const void *)(a.res_out + base) : (const void *)a.gamma,
               RES_OUT ? a.c16 * 16 : 0);
  if constexpr (RES_OUT) {
    // After every load has arrived (gamma comes last), so that no later wait
    // for a load has to wait for this store as well.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    if (valid) buf_store16<false>(rout, (first + t) * 16, hv);
  }

  float pss, pmx;
  block_pair(ss, mx, red, 0, wave, nwaves, pss, pmx);

  // Publish this part's pair; part 0 also raises the unused slots.
  if (t == 0) {
    __hip_atomic_store(slots + 2 * part, ws_word(count, pss), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(slots + 2 * part + 1, ws_word(count, pmx), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    if (part == 0) {
      for (int s = a.parts; s < kSplitSlots; ++s) {
        __hip_atomic_store(slots + 2 * s, ws_word(count, 0.0f), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(slots + 2 * s + 1, ws_word(count, 0.0f), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  // Gather: lane j polls part j's words, a bounded number of times.
  if (t < a.parts) {
    float sj = pss, mj = pmx;
    int miss = 0;
    if (t != part) {
      miss = 1;
      for (int polls = 0; polls <= a.spin_polls; ++polls) {
        const unsigned long long w0 =
            __hip_atomic_load(slots + 2 * t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const unsigned long long w1 =
            __hip_atomic_load(slots + 2 * t + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (ws_count(w0) == count && ws_count(w1) == count) {
          sj = ws_value(w0);
          mj = ws_value(w1);
          miss = 0;
          break;
        }
      }
    }
    part_ss[t] = sj;
    part_mx[t] = mj;
    missing[t] = miss;
  }
  __syncthreads();

  // A partner that did not publish in time: its pair, computed here exactly
  // as the partner computes it (same lanes, chunks and reduction order).
  int slot = 1;
  for (int j = 0; j < a.parts; ++j) {
    if (missing[j]) {  // workgroup-uniform: read from LDS after a barrier
      const int fj = j * a.cpp;
      const bool vj = t < a.cpp && fj + t <= last;
      ChunkIn<P, RES_IN> inj;
      split_load<P, RES_IN>(a, base, min(fj + t, last), inj);
      __builtin_amdgcn_sched_barrier(0);
      u32x4 hvj;
      float hgj[8];
      float ssj = 0.0f, mxj = 0.0f;
      split_chunk<P, RES_IN>(a, inj, vj, hvj, hgj, ssj, mxj);
      float tj, mj;
      block_pair(ssj, mxj, red, slot, wave, nwaves, tj, mj);
      slot ^= 1;
      if (t == 0) {
        part_ss[j] = tj;
        part_mx[j] = mj;
      }
      __syncthreads();
    }
  }

  // The row's statistics: the parts' pairs in part order.
  float tot = 0.0f, m = 0.0f;
  for (int j = 0; j < a.parts; ++j) {
    tot += part_ss[j];
    m = max_nonneg(m, part_mx[j]);
  }
  const float den = tot * a.inv_cols + a.eps;
  const float r = den > 0.0f ? __builtin_amdgcn_rsqf(den) : 0.0f;
  const float amax = m * r;
  const float scale = fmaxf(fminf(amax, a.ub) / 448.0f, fmt_floor<kFmtE4m3>());
  const float cq = r * __builtin_amdgcn_rcpf(scale);
  if (part == 0 && t == 0) a.scales[row] = scale;

  float q[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) q[e] = fminf(fmaxf(hg[e] * cq, -448.0f), 448.0f);
  const __amdgpu_buffer_rsrc_t qout = row_rsrc(a.out + base, a.c16 * 8);
  if (valid) buf_store8<false>(qout, (first + t) * 8, pack_e4m3(q));
}

namespace {

template <int P>
SplitKernel split_by_res(bool res_in, bool res_out) {
  if (res_in)
    return res_out ? arnfp8_split_kernel<P, true, true> : arnfp8_split_kernel<P, true, false>;
  return res_out ? arnfp8_split_kernel<P, false, true> : arnfp8_split_kernel<P, false, false>;
}

}  // namespace

SplitKernel split_table(int P, bool res_in, bool res_out) {
  switch (P) {
    case 1: return split_by_res<1>(res_in, res_out);
    case 2: return split_by_res<2>(res_in, res_out);
    case 3: return split_by_res<3>(res_in, res_out);
    case 4: return split_by_res<4>(res_in, res_out);
    case 5: return split_by_res<5>(res_in, res_out);
    case 6: return split_by_res<6>(res_in, res_out);
    case 7: return split_by_res<7>(res_in, res_out);
    default: return split_by_res<8>(res_in, res_out);
  }
}

}  // namespace arnfp8
