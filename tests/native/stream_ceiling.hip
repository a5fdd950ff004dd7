// What plain streaming kernels reach on this GPU for the read/write mixes of
// the row kernels, as the reference point for their HBM rooflines: read only,
// one read per write (the forwards: x in, y out) and two reads per write (the
// backwards: x and dy in, dx out).  256 MiB per operand, the size of one
// 16384 x 8192 bf16 tensor.  Every access is a 16-byte vector load or store
// with the nontemporal policy, as in the row kernels; each mix is timed over
// grid-stride loops of several grid, block and unroll sizes and over a
// row-chunked walk like the row kernels', and the best is kept.  "hot":
// launches back to back; "cold": each launch after a 1 GiB write to other
// memory.
//
// Prints one JSON line.  Run by bench.py (before it touches the GPU itself)
// and usable on its own: tests/native/bin/stream_ceiling
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <string>
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

// Grid-stride over n 16-byte vectors, UNROLL loads of each input in flight
// per thread.  Every index is below n (the loop condition covers the last
// unrolled access); n is a multiple of UNROLL * stride for the shapes used,
// so every vector is visited.
template <int UNROLL, int READS, bool WRITE>
__global__ void stream_kernel(const u32x4* __restrict__ a, const u32x4* __restrict__ b, u32x4* __restrict__ c,
                              u32x4* __restrict__ sink, long n) {
  const long stride = static_cast<long>(gridDim.x) * blockDim.x;
  const long first = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (long i = first; i + (UNROLL - 1) * stride < n; i += UNROLL * stride) {
    u32x4 v[UNROLL], w[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      v[u] = __builtin_nontemporal_load(a + i + u * stride);
      if (READS == 2) w[u] = __builtin_nontemporal_load(b + i + u * stride);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const u32x4 r = READS == 2 ? (v[u] ^ w[u]) : v[u];
      if (WRITE) {
        __builtin_nontemporal_store(r, c + i + u * stride);
      } else {
        acc ^= r;
      }
    }
  }
  if (!WRITE) sink[first] = acc;  // keeps the loads; one vector per thread
}

// Row-chunked, as the row kernels walk their tensors: rows of 1024 vectors
// (16 KiB), 512 threads x 2 vectors per row, workgroup b taking rows b,
// b + grid, ...  Every index is below rows * 1024.
template <int READS, bool WRITE>
__global__ void rows_kernel(const u32x4* __restrict__ a, const u32x4* __restrict__ b, u32x4* __restrict__ c,
                            u32x4* __restrict__ sink, long rows) {
  constexpr int kRowVecs = 1024;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (long r = blockIdx.x; r < rows; r += gridDim.x) {
    const long base = r * kRowVecs + threadIdx.x;
    u32x4 v[2], w[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      v[u] = __builtin_nontemporal_load(a + base + u * 512);
      if (READS == 2) w[u] = __builtin_nontemporal_load(b + base + u * 512);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const u32x4 x = READS == 2 ? (v[u] ^ w[u]) : v[u];
      if (WRITE) {
        __builtin_nontemporal_store(x, c + base + u * 512);
      } else {
        acc ^= x;
      }
    }
  }
  if (!WRITE) sink[static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x] = acc;
}

struct Result {
  double hot = 0, cold = 0;
  char shape[48] = "";
  std::string all;  // "shape": hot GB/s, for every shape timed
};

int main() {
  const long bytes = 256L << 20;
  const long n = bytes / 16;
  const long flush_bytes = 1L << 30;
  const int grids[] = {256, 512, 1024};
  const int blocks[] = {256, 512};
  const int row_grids[] = {512, 2048, 16384};
  const long rows = n / 1024;
  u32x4 *a, *b, *c, *sink;
  void* flush;
  CHECK(hipMalloc(&a, bytes));
  CHECK(hipMalloc(&b, bytes));
  CHECK(hipMalloc(&c, bytes));
  CHECK(hipMalloc(&sink, 16384L * 512 * 16));  // one vector per thread of the largest grid
  CHECK(hipMalloc(&flush, flush_bytes));
  CHECK(hipMemset(a, 1, bytes));
  CHECK(hipMemset(b, 2, bytes));
  CHECK(hipMemset(c, 0, bytes));
  hipEvent_t t0, t1;
  CHECK(hipEventCreate(&t0));
  CHECK(hipEventCreate(&t1));

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
    for (int k = 0; k < 7; ++k) {
      CHECK(hipMemsetAsync(flush, k, flush_bytes));
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
    char item[96];
    std::snprintf(item, sizeof item, "%s\"%s\": %.0f", best.all.empty() ? "" : ", ", shape, hot);
    best.all += item;
    best.cold = std::max(best.cold, cold);
  };

  Result read, copy, r2w1;
  char shape[48];
  for (int g : grids)
    for (int bs : blocks) {
      std::snprintf(shape, sizeof shape, "grid-stride x4, %d x %d", g, bs);
      measure([&] { stream_kernel<4, 1, false><<<g, bs>>>(a, b, c, sink, n); }, 1.0, read, shape);
      measure([&] { stream_kernel<4, 1, true><<<g, bs>>>(a, b, c, sink, n); }, 2.0, copy, shape);
      measure([&] { stream_kernel<4, 2, true><<<g, bs>>>(a, b, c, sink, n); }, 3.0, r2w1, shape);
      std::snprintf(shape, sizeof shape, "grid-stride x2, %d x %d", g, bs);
      measure([&] { stream_kernel<2, 1, true><<<g, bs>>>(a, b, c, sink, n); }, 2.0, copy, shape);
      measure([&] { stream_kernel<2, 2, true><<<g, bs>>>(a, b, c, sink, n); }, 3.0, r2w1, shape);
    }
  for (int g : row_grids) {
    std::snprintf(shape, sizeof shape, "16 KiB rows, %d x 512", g);
    measure([&] { rows_kernel<1, false><<<g, 512>>>(a, b, c, sink, rows); }, 1.0, read, shape);
    measure([&] { rows_kernel<1, true><<<g, 512>>>(a, b, c, sink, rows); }, 2.0, copy, shape);
    measure([&] { rows_kernel<2, true><<<g, 512>>>(a, b, c, sink, rows); }, 3.0, r2w1, shape);
  }
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  auto obj = [](const Result& r) {
    char head[160];
    std::snprintf(head, sizeof head, "{\"hot_gbps\": %.0f, \"cold_gbps\": %.0f, \"best_hot_shape\": \"%s\", ", r.hot,
                  r.cold, r.shape);
    return std::string(head) + "\"hot_gbps_by_shape\": {" + r.all + "}}";
  };
  std::printf("{\"bytes_per_operand\": %ld, \"read\": %s, \"read1_write1\": %s, \"read2_write1\": %s}\n", bytes,
              obj(read).c_str(), obj(copy).c_str(), obj(r2w1).c_str());
  CHECK(hipFree(a));
  CHECK(hipFree(b));
  CHECK(hipFree(c));
  CHECK(hipFree(sink));
  CHECK(hipFree(flush));
  return 0;
}
