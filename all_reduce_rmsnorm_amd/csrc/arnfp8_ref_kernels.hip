// arnfp8_ref_kernels.hip -- achievable-bandwidth reference kernels for the
// benchmark (built into libarnfp8_ref.so, apart from the product library).
//
// They move the fused epilogue's bytes with none of its arithmetic, in its
// access pattern: one workgroup per row (rows walked grid-stride), lane t of a
// T-lane workgroup owning the row's 16-byte chunks t, t + T, ..., every global
// access a 16-byte vector (non-temporal loads, non-temporal buffer stores).
// Measured beside the fused kernel they bound what its byte mix can reach on
// the device:
//   arnref_read   S read streams of [rows, row_bytes]; one 16-byte word of
//                 XOR per row is written so that the loads cannot be dropped.
//   arnref_write  W write streams of [rows, row_bytes], a constant pattern.
//   arnref_twin   the fused kernel's byte mix: S read streams of 16 bytes per
//                 chunk, and per chunk one 16-byte and one 8-byte store (the
//                 updated residual and the fp8 row), each the XOR of the
//                 chunk's loads (so every store waits for its loads, as in
//                 the fused kernel), no other arithmetic.
//   arnref_empty  a kernel that does nothing, on the grid of one workgroup per
//                 row: the cost of a launch alone.
//   arnref_exchange  the cost of one exchange between workgroups: groups of S
//                 workgroups each publish one 64-bit word (a 32-bit payload and
//                 a 32-bit count) with a relaxed device-scope atomic store and
//                 wait, one lane per partner, until every partner's word
//                 carries the same count, as a
//                 row split across S workgroups would trade its row statistics.
//                 Each word has a single writer whose count goes up by one per
//                 launch, so partners stay in step across launches and graph
//                 replays with no host-side epoch.  The wait is bounded
//                 (kSpinLimit polls); a wait that runs out is counted in
//                 `timeouts` and the workgroup goes on, so every launch ends.
// Shapes follow the fused kernel: lanes = T, chunks per lane = V, T * V * 16
// >= row_bytes; up to 1024 lanes with one chunk per lane, else up to 512.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxStreams = 10;
constexpr int kStoreNt = 2;
constexpr int kRawBufferWord3 = 0x00020000;

struct Streams {
  const u32x4 *p[kMaxStreams];
};
struct OutStreams {
  u32x4 *p[kMaxStreams];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, kRawBufferWord3);
}

template <int S, int V>
__global__ __launch_bounds__(V == 1 ? 1024 : 512) void read_kernel(Streams in, u32x4 *__restrict__ sink,
                                                   int64_t rows, int c16) {
  const int t = threadIdx.x, T = blockDim.x, last = c16 - 1;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const int64_t base = row * (int64_t)c16;
    u32x4 acc = {0, 0, 0, 0};
    u32x4 x[V][S];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int c = min(v * T + t, last);
#pragma unroll
      for (int s = 0; s < S; ++s) x[v][s] = __builtin_nontemporal_load(in.p[s] + base + c);
    }
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int s = 0; s < S; ++s) acc ^= x[v][s];
    // Every lane tests its own XOR against a constant that random data
    // essentially never produces: the loads of every lane stay live, and
    // (almost) nothing is written.
    if ((acc.x | acc.y | acc.z | acc.w) == 0x9E3779B9u) sink[row] = acc;
  }
}

template <int W, int V>
__global__ __launch_bounds__(V == 1 ? 1024 : 512) void write_kernel(OutStreams out, int64_t rows, int c16) {
  const int t = threadIdx.x, T = blockDim.x, last = c16 - 1;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const int64_t base = row * (int64_t)c16;
    const u32x4 val = {(uint32_t)row, (uint32_t)t, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int c = v * T + t;
      if (c <= last) {
#pragma unroll
        for (int w = 0; w < W; ++w)
          __builtin_amdgcn_raw_buffer_store_b128(val, rsrc(out.p[w] + base, c16 * 16), c * 16, 0,
                                                 kStoreNt);
      }
    }
  }
}

template <int S, int V>
__global__ __launch_bounds__(V == 1 ? 1024 : 512) void twin_kernel(Streams in, u32x4 *__restrict__ out16,
                                                   u32x2 *__restrict__ out8, int64_t rows,
                                                   int c16) {
  const int t = threadIdx.x, T = blockDim.x, last = c16 - 1;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const int64_t base = row * (int64_t)c16;
    const __amdgpu_buffer_rsrc_t r16 = rsrc(out16 + base, c16 * 16);
    const __amdgpu_buffer_rsrc_t r8 = rsrc(out8 + base, c16 * 8);
    u32x4 x[V][S];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int c = min(v * T + t, last);
#pragma unroll
      for (int s = 0; s < S; ++s) x[v][s] = __builtin_nontemporal_load(in.p[s] + base + c);
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
      u32x4 acc = x[v][0];
#pragma unroll
      for (int s = 1; s < S; ++s) acc ^= x[v][s];
      const int c = v * T + t;
      if (c <= last) {
        __builtin_amdgcn_raw_buffer_store_b128(acc, r16, c * 16, 0, kStoreNt);
        __builtin_amdgcn_raw_buffer_store_b64((u32x2){acc.x ^ acc.z, acc.y ^ acc.w}, r8, c * 8, 0,
                                              kStoreNt);
      }
    }
  }
}

__global__ __launch_bounds__(1024) void empty_kernel(int64_t rows) {}

constexpr int kSpinLimit = 1 << 16;

// Workgroup b belongs to group b / S (consecutive ids) or, with `stride` 8,
// to the group of ids that agree modulo 8 (workgroups are dispatched to the
// eight XCDs in turn, so such a group shares one XCD and its L2).
__global__ __launch_bounds__(64) void exchange_kernel(unsigned long long *words, int S, int stride,
                                                      unsigned *timeouts) {
  const int b = blockIdx.x;
  int first, step;
  if (stride == 8) {
    const int lane8 = b % 8, k = b / 8;  // k-th workgroup on its XCD
    first = (k / S) * S * 8 + lane8;
    step = 8;
  } else {
    first = (b / S) * S;
    step = 1;
  }
  // Lane 0 publishes; lane j < S then polls partner j, all partners at once.
  unsigned long long *mine = words + b;
  const unsigned long long old = __hip_atomic_load(mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned count = (unsigned)(old >> 32) + 1u;
  if (threadIdx.x == 0) {
    const unsigned long long word = ((unsigned long long)count << 32) | (unsigned)b;
    __hip_atomic_store(mine, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const int j = threadIdx.x;
  if (j < S) {
    unsigned long long *theirs = words + first + j * step;
    if (theirs != mine) {
      int spins = 0;
      while ((unsigned)(__hip_atomic_load(theirs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >>
                        32) != count) {
        if (++spins == kSpinLimit) {
          atomicAdd(timeouts, 1u);
          break;
        }
      }
    }
  }
}

typedef void (*ReadK)(Streams, u32x4 *, int64_t, int);
typedef void (*WriteK)(OutStreams, int64_t, int);
typedef void (*TwinK)(Streams, u32x4 *, u32x2 *, int64_t, int);

template <int V>
ReadK read_by_s(int s) {
  switch (s) {
    case 1: return read_kernel<1, V>;
    case 5: return read_kernel<5, V>;
    case 9: return read_kernel<9, V>;
    default: return nullptr;
  }
}
ReadK read_table(int s, int v) {
  switch (v) {
    case 1: return read_by_s<1>(s);
    case 2: return read_by_s<2>(s);
    case 4: return read_by_s<4>(s);
    default: return nullptr;
  }
}
WriteK write_table(int w, int v) {
  if (w == 1) return v == 1 ? write_kernel<1, 1> : v == 2 ? write_kernel<1, 2> : nullptr;
  if (w == 2) return v == 1 ? write_kernel<2, 1> : v == 2 ? write_kernel<2, 2> : nullptr;
  return nullptr;
}
template <int V>
TwinK twin_by_s(int s) {
  switch (s) {
    case 5: return twin_kernel<5, V>;
    case 9: return twin_kernel<9, V>;
    default: return nullptr;
  }
}
TwinK twin_table(int s, int v) {
  switch (v) {
    case 1: return twin_by_s<1>(s);
    case 2: return twin_by_s<2>(s);
    default: return nullptr;
  }
}

// Lanes and chunks per lane: the given ones, or 0 for the fused kernel's
// choice for this row (the smallest of 1, 2, 4 chunks that fits 512 lanes).
bool shape(int c16, int *threads, int *vpt) {
  if (*vpt == 0) *vpt = c16 <= 512 ? 1 : (c16 <= 1024 ? 2 : 4);
  if (*threads == 0) *threads = ((c16 + *vpt - 1) / *vpt + 63) / 64 * 64;
  return *threads >= 64 && *threads <= (*vpt == 1 ? 1024 : 512) && *threads % 64 == 0 &&
         (int64_t)*threads * *vpt >= c16;
}

bool sane(int64_t rows, int64_t row_bytes) {
  return rows > 0 && row_bytes > 0 && row_bytes % 16 == 0 && row_bytes / 16 <= 4096;
}

template <typename... Args>
int launch(void (*k)(Args...), int64_t rows, int threads, hipStream_t stream, Args... args) {
  void *argv[] = {(void *)&args...};
  const unsigned grid = (unsigned)(rows < 65536 ? rows : 65536);
  return hipLaunchKernel((const void *)k, dim3(grid), dim3(threads), argv, 0, stream) == hipSuccess
             ? 0
             : 6;
}

}  // namespace

// Each returns 0, 3 for a bad size or shape, 4 for an unsupported stream
// count, or 6 when the launch fails.  Pointers are 16-byte aligned device
// memory of rows * row_bytes bytes per stream (sink: rows * 16 bytes).
extern "C" int arnref_read(const void *const *streams, int nstreams, void *sink, int64_t rows,
                           int64_t row_bytes, int threads, int vpt, hipStream_t stream) {
  if (!sane(rows, row_bytes)) return 3;
  const int c16 = (int)(row_bytes / 16);
  if (!shape(c16, &threads, &vpt)) return 3;
  ReadK k = read_table(nstreams, vpt);
  if (k == nullptr) return 4;
  Streams s;
  for (int i = 0; i < kMaxStreams; ++i) s.p[i] = (const u32x4 *)streams[i < nstreams ? i : 0];
  return launch(k, rows, threads, stream, s, (u32x4 *)sink, rows, c16);
}

extern "C" int arnref_write(void *const *outs, int nouts, int64_t rows, int64_t row_bytes,
                            int threads, int vpt, hipStream_t stream) {
  if (!sane(rows, row_bytes)) return 3;
  const int c16 = (int)(row_bytes / 16);
  if (!shape(c16, &threads, &vpt)) return 3;
  WriteK k = write_table(nouts, vpt);
  if (k == nullptr) return 4;
  OutStreams o;
  for (int i = 0; i < kMaxStreams; ++i) o.p[i] = (u32x4 *)outs[i < nouts ? i : 0];
  return launch(k, rows, threads, stream, o, rows, c16);
}

extern "C" int arnref_twin(const void *const *streams, int nstreams, void *out16, void *out8,
                           int64_t rows, int64_t row_bytes, int threads, int vpt,
                           hipStream_t stream) {
  if (!sane(rows, row_bytes)) return 3;
  const int c16 = (int)(row_bytes / 16);
  if (!shape(c16, &threads, &vpt)) return 3;
  TwinK k = twin_table(nstreams, vpt);
  if (k == nullptr) return 4;
  Streams s;
  for (int i = 0; i < kMaxStreams; ++i) s.p[i] = (const u32x4 *)streams[i < nstreams ? i : 0];
  return launch(k, rows, threads, stream, s, (u32x4 *)out16, (u32x2 *)out8, rows, c16);
}

extern "C" int arnref_empty(int64_t rows, int threads, hipStream_t stream) {
  if (rows <= 0 || threads < 64 || threads > 1024 || threads % 64) return 3;
  return launch(empty_kernel, rows, threads, stream, rows);
}

// words: nwg zero-initialised 64-bit words, untouched by anything else;
// timeouts: one 32-bit counter.  nwg must be a multiple of S (and of 8 * S
// with stride 8); every workgroup of the grid must be resident at once (the
// bench launches at most one 64-lane workgroup per CU).
extern "C" int arnref_exchange(void *words, int nwg, int S, int stride, void *timeouts,
                               hipStream_t stream) {
  if (words == nullptr || timeouts == nullptr || S < 1 || S > 64 || nwg < S || nwg > 4096 ||
      (stride != 1 && stride != 8) || nwg % (S * (stride == 8 ? 8 : 1)) != 0)
    return 3;
  unsigned long long *w = (unsigned long long *)words;
  unsigned *t = (unsigned *)timeouts;
  void *argv[] = {&w, &S, &stride, &t};
  return hipLaunchKernel((const void *)exchange_kernel, dim3((unsigned)nwg), dim3(64), argv, 0,
                         stream) == hipSuccess
             ? 0
             : 6;
}
