// What plain streaming kernels reach on this GPU for the read/write mixes of
// the row kernels, as the reference point for their HBM rooflines: read only,
// one read per write (the forwards: x in, y out), two reads per write (the
// backwards: x and dy in, dx out) and two reads per write in place (dx over
// dy, as in the headline backward), and three reads with three writes (the
// elementwise SwiGLU backward).  256 MiB per
// operand, the size of one 16384 x 8192 bf16 tensor.  Every access is a
// 16-byte vector load or store.
// The search covers, for every mix:
//   * grid-stride loops: 32, 64 or 128 bytes of each input in flight per lane
//     (2, 4 or 8 vectors), 256-, 512- and 1024-thread workgroups, grids of
//     256 to 4096 workgroups;
//   * row walks as the row kernels walk their tensors: rows of 16 KiB, 256-,
//     512- or 1024-thread workgroups holding a row in 4, 2 or 1 vectors per
//     lane (all of a row's loads before its stores), workgroup b taking rows
//     b, b + grid, ...; persistent grids of 256 to 2048 workgroups and one
//     row per workgroup (16384);
// each with the nontemporal policy (as in the row kernels) and the default
// one, and keeps the best.  "hot": launches back to back; "cold": each launch
// after a 1 GiB write to other memory and a read of it (so no dirty line of
// the write is left to be written back inside the timed launch).
//
// Prints one JSON line.  Run by bench.py (before it touches the GPU itself)
// and usable on its own: tests/native/bin/stream_ceiling
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <type_traits>
#include <vector>

#define CHECK(x)                                                                            \
  do {                                                                                      \
    hipError_t e_ = (x);                                                                    \
    if (e_ != hipSuccess) {                                                                 \
      std::fprintf(stderr, "stream_ceiling: %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      std::exit(1);                                                                         \
    }                                                                                       \
  } while (0)

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ u32x4 load(const u32x4* p) {
  if constexpr (NT) {
    return __builtin_nontemporal_load(p);
  } else {
    return *p;
  }
}

template <bool NT>
__device__ __forceinline__ void store(u32x4* p, u32x4 v) {
  if constexpr (NT) {
    __builtin_nontemporal_store(v, p);
  } else {
    *p = v;
  }
}

// Grid-stride over n 16-byte vectors, UNROLL loads of each input in flight
// per thread.  Every index is below n (the loop condition covers the last
// unrolled access); n is a multiple of UNROLL * stride for the shapes used
// (powers of two, UNROLL * stride <= n), so every vector is visited.  c may
// equal b.
template <int UNROLL, int READS, bool WRITE, bool NT>
__global__ void stream_kernel(const u32x4* a, const u32x4* b, u32x4* c, u32x4* __restrict__ sink, long n) {
  const long stride = static_cast<long>(gridDim.x) * blockDim.x;
  const long first = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (long i = first; i + (UNROLL - 1) * stride < n; i += UNROLL * stride) {
    u32x4 v[UNROLL], w[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      v[u] = load<NT>(a + i + u * stride);
      if (READS == 2) w[u] = load<NT>(b + i + u * stride);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const u32x4 r = READS == 2 ? (v[u] ^ w[u]) : v[u];
      if (WRITE) {
        store<NT>(c + i + u * stride, r);
      } else {
        acc ^= r;
      }
    }
  }
  if (!WRITE) sink[first] = acc;  // keeps the loads; one vector per thread
}

// Three reads, three writes: grid-stride as stream_kernel (the same index
// bounds), each output a different function of the three inputs.
template <int UNROLL, bool NT>
__global__ void stream3_kernel(const u32x4* a, const u32x4* b, const u32x4* c, u32x4* d, u32x4* e, u32x4* f,
                               long n) {
  const long stride = static_cast<long>(gridDim.x) * blockDim.x;
  const long first = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  for (long i = first; i + (UNROLL - 1) * stride < n; i += UNROLL * stride) {
    u32x4 v[UNROLL], w[UNROLL], x[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      v[u] = load<NT>(a + i + u * stride);
      w[u] = load<NT>(b + i + u * stride);
      x[u] = load<NT>(c + i + u * stride);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      store<NT>(d + i + u * stride, v[u] ^ w[u]);
      store<NT>(e + i + u * stride, w[u] + x[u]);
      store<NT>(f + i + u * stride, x[u] | v[u]);
    }
  }
}

// Row walk: rows of kRowVecs vectors (16 KiB), a T-thread workgroup covering
// a row with kRowVecs / T vectors per lane, all of them loaded before any is
// stored; workgroup b takes rows b, b + grid, ...  Every index is below
// rows * kRowVecs.  c may equal b (each lane reads its own vectors of b
// before it writes them).
constexpr int kRowVecs = 1024;
template <int T, int READS, bool WRITE, bool NT>
__global__ __launch_bounds__(T) void rows_kernel(const u32x4* a, const u32x4* b, u32x4* c, u32x4* __restrict__ sink,
                                                 long rows) {
  constexpr int kPer = kRowVecs / T;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (long r = blockIdx.x; r < rows; r += gridDim.x) {
    const long base = r * kRowVecs + threadIdx.x;
    u32x4 v[kPer], w[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      v[u] = load<NT>(a + base + u * T);
      if (READS == 2) w[u] = load<NT>(b + base + u * T);
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const u32x4 x = READS == 2 ? (v[u] ^ w[u]) : v[u];
      if (WRITE) {
        store<NT>(c + base + u * T, x);
      } else {
        acc ^= x;
      }
    }
  }
  if (!WRITE) sink[static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x] = acc;
}

// Three reads, three writes over the same row walk.
template <int T, bool NT>
__global__ __launch_bounds__(T) void rows3_kernel(const u32x4* a, const u32x4* b, const u32x4* c, u32x4* d, u32x4* e,
                                                  u32x4* f, long rows) {
  constexpr int kPer = kRowVecs / T;
  for (long r = blockIdx.x; r < rows; r += gridDim.x) {
    const long base = r * kRowVecs + threadIdx.x;
    u32x4 v[kPer], w[kPer], x[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      v[u] = load<NT>(a + base + u * T);
      w[u] = load<NT>(b + base + u * T);
      x[u] = load<NT>(c + base + u * T);
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      store<NT>(d + base + u * T, v[u] ^ w[u]);
      store<NT>(e + base + u * T, w[u] + x[u]);
      store<NT>(f + base + u * T, x[u] | v[u]);
    }
  }
}

struct Result {
  double hot = 0, cold = 0;
  char shape[64] = "";
  std::string all;  // "shape": hot GB/s, for every shape timed
};

// The mixes: input count, output count, whether the output is the second input.
enum Mix { kRead, kCopy, kR2W1, kR2W1InPlace, kR3W3, kMixes };

int main() {
  const long bytes = 256L << 20;
  const long n = bytes / 16;
  const long rows = n / kRowVecs;
  const long flush_bytes = 1L << 30;
  const int grids[] = {256, 512, 1024, 2048, 4096};
  const int row_grids[] = {256, 512, 1024, 2048, 16384};
  u32x4 *a, *b, *c, *d, *e, *f, *sink, *flush;
  CHECK(hipMalloc(&a, bytes));
  CHECK(hipMalloc(&b, bytes));
  CHECK(hipMalloc(&c, bytes));
  CHECK(hipMalloc(&d, bytes));
  CHECK(hipMalloc(&e, bytes));
  CHECK(hipMalloc(&f, bytes));
  // one vector per thread of the largest grid of either kind
  const long sink_vecs = std::max(4096L * 1024, 16384L * 1024);
  CHECK(hipMalloc(&sink, sink_vecs * 16));
  CHECK(hipMalloc(&flush, flush_bytes));
  CHECK(hipMemset(a, 1, bytes));
  CHECK(hipMemset(b, 2, bytes));
  CHECK(hipMemset(c, 0, bytes));
  CHECK(hipMemset(d, 0, bytes));
  CHECK(hipMemset(e, 0, bytes));
  CHECK(hipMemset(f, 0, bytes));
  hipEvent_t t0, t1;
  CHECK(hipEventCreate(&t0));
  CHECK(hipEventCreate(&t1));
  const long flush_n = flush_bytes / 16;

  // bytes moved per launch: (reads + writes) operands of `bytes`
  auto measure = [&](auto launch, double operands, Result& best, const char* shape) {
    for (int k = 0; k < 5; ++k) launch();  // ramp
    CHECK(hipDeviceSynchronize());
    const int reps = 20;
    CHECK(hipEventRecord(t0));
    for (int k = 0; k < reps; ++k) launch();
    CHECK(hipEventRecord(t1));
    CHECK(hipEventSynchronize(t1));
    float ms = 0;
    CHECK(hipEventElapsedTime(&ms, t0, t1));
    const double hot = operands * bytes / (ms / reps * 1e-3) / 1e9;
    std::vector<float> cold_ms;
    for (int k = 0; k < 5; ++k) {
      CHECK(hipMemsetAsync(flush, k, flush_bytes));
      // 4096 x 256 threads x 4 vectors: flush_n is a multiple of that stride
      stream_kernel<4, 1, false, false><<<4096, 256>>>(flush, flush, flush, sink, flush_n);
      CHECK(hipEventRecord(t0));
      launch();
      CHECK(hipEventRecord(t1));
      CHECK(hipEventSynchronize(t1));
      CHECK(hipEventElapsedTime(&ms, t0, t1));
      cold_ms.push_back(ms);
    }
    std::sort(cold_ms.begin(), cold_ms.end());
    const double cold = operands * bytes / (cold_ms[cold_ms.size() / 2] * 1e-3) / 1e9;
    if (hot > best.hot) {
      best.hot = hot;
      std::snprintf(best.shape, sizeof best.shape, "%s", shape);
    }
    char item[112];
    std::snprintf(item, sizeof item, "%s\"%s\": %.0f", best.all.empty() ? "" : ", ", shape, hot);
    best.all += item;
    best.cold = std::max(best.cold, cold);
  };

  Result res[kMixes];
  char shape[64];
  // one grid-stride shape for every mix, at one policy
  auto stride_shapes = [&](auto unroll_tag, auto nt_tag, int g, int bs) {
    constexpr int U = decltype(unroll_tag)::value;
    constexpr bool NT = decltype(nt_tag)::value;
    if (static_cast<long>(U) * g * bs > n) return;
    const char* pol = NT ? "nt" : "default";
    std::snprintf(shape, sizeof shape, "grid-stride %d B/lane, %d x %d, %s", U * 16, g, bs, pol);
    measure([&] { stream_kernel<U, 1, false, NT><<<g, bs>>>(a, b, c, sink, n); }, 1.0, res[kRead], shape);
    measure([&] { stream_kernel<U, 1, true, NT><<<g, bs>>>(a, b, c, sink, n); }, 2.0, res[kCopy], shape);
    measure([&] { stream_kernel<U, 2, true, NT><<<g, bs>>>(a, b, c, sink, n); }, 3.0, res[kR2W1], shape);
    measure([&] { stream_kernel<U, 2, true, NT><<<g, bs>>>(a, b, b, sink, n); }, 3.0, res[kR2W1InPlace], shape);
    measure([&] { stream3_kernel<U, NT><<<g, bs>>>(a, b, c, d, e, f, n); }, 6.0, res[kR3W3], shape);
  };
  auto row_shapes = [&](auto t_tag, auto nt_tag, int g) {
    constexpr int T = decltype(t_tag)::value;
    constexpr bool NT = decltype(nt_tag)::value;
    const char* pol = NT ? "nt" : "default";
    std::snprintf(shape, sizeof shape, "16 KiB rows, %d x %d (%d vectors per lane), %s", g, T, kRowVecs / T, pol);
    measure([&] { rows_kernel<T, 1, false, NT><<<g, T>>>(a, b, c, sink, rows); }, 1.0, res[kRead], shape);
    measure([&] { rows_kernel<T, 1, true, NT><<<g, T>>>(a, b, c, sink, rows); }, 2.0, res[kCopy], shape);
    measure([&] { rows_kernel<T, 2, true, NT><<<g, T>>>(a, b, c, sink, rows); }, 3.0, res[kR2W1], shape);
    measure([&] { rows_kernel<T, 2, true, NT><<<g, T>>>(a, b, b, sink, rows); }, 3.0, res[kR2W1InPlace], shape);
    measure([&] { rows3_kernel<T, NT><<<g, T>>>(a, b, c, d, e, f, rows); }, 6.0, res[kR3W3], shape);
  };
  using nt = std::true_type;
  using dflt = std::false_type;
  for (int g : grids)
    for (int bs : {256, 512, 1024}) {
      stride_shapes(std::integral_constant<int, 2>{}, nt{}, g, bs);
      stride_shapes(std::integral_constant<int, 4>{}, nt{}, g, bs);
      stride_shapes(std::integral_constant<int, 8>{}, nt{}, g, bs);
      stride_shapes(std::integral_constant<int, 2>{}, dflt{}, g, bs);
      stride_shapes(std::integral_constant<int, 4>{}, dflt{}, g, bs);
      stride_shapes(std::integral_constant<int, 8>{}, dflt{}, g, bs);
    }
  for (int g : row_grids) {
    row_shapes(std::integral_constant<int, 256>{}, nt{}, g);
    row_shapes(std::integral_constant<int, 512>{}, nt{}, g);
    row_shapes(std::integral_constant<int, 1024>{}, nt{}, g);
    row_shapes(std::integral_constant<int, 256>{}, dflt{}, g);
    row_shapes(std::integral_constant<int, 512>{}, dflt{}, g);
    row_shapes(std::integral_constant<int, 1024>{}, dflt{}, g);
  }
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  auto obj = [](const Result& r) {
    char head[200];
    std::snprintf(head, sizeof head, "{\"hot_gbps\": %.0f, \"cold_gbps\": %.0f, \"best_hot_shape\": \"%s\", ", r.hot,
                  r.cold, r.shape);
    return std::string(head) + "\"hot_gbps_by_shape\": {" + r.all + "}}";
  };
  std::printf(
      "{\"bytes_per_operand\": %ld, \"read\": %s, \"read1_write1\": %s, \"read2_write1\": %s, "
      "\"read2_write1_in_place\": %s, \"read3_write3\": %s}\n",
      bytes, obj(res[kRead]).c_str(), obj(res[kCopy]).c_str(), obj(res[kR2W1]).c_str(),
      obj(res[kR2W1InPlace]).c_str(), obj(res[kR3W3]).c_str());
  CHECK(hipFree(a));
  CHECK(hipFree(b));
  CHECK(hipFree(c));
  CHECK(hipFree(d));
  CHECK(hipFree(e));
  CHECK(hipFree(f));
  CHECK(hipFree(sink));
  CHECK(hipFree(flush));
  return 0;
}
