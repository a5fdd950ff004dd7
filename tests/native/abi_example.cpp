// A plain C++ caller of the C ABI (no Python, no PyTorch): one row of fp32
// data through rmsnorm_fwd and rmsnorm_bwd on the GPU, with device memory from
// hipMalloc and the null stream.  The values come from the command line,
//   abi_example N eps gemma x_0..x_{N-1} gamma_0.. dy_0..
// and the outputs are printed as "y ...", "r ...", "dx ...", "dgamma ...";
// tests/test_c_abi_gpu.py feeds it the worked examples kept in tests/golden/
// and compares what it prints.  It also checks that a contract violation is
// reported as a status and launches nothing.  Exit status 0 on success.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

#include "rmsnorm.h"

#define CHECK_HIP(e)                                                         \
  do {                                                                       \
    hipError_t err_ = (e);                                                   \
    if (err_ != hipSuccess) {                                                \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(err_), __LINE__); \
      return 2;                                                              \
    }                                                                        \
  } while (0)

static void print_row(const char* name, const std::vector<float>& v) {
  std::printf("%s", name);
  for (float f : v) std::printf(" %.9g", f);
  std::printf("\n");
}

int main(int argc, char** argv) {
  if (argc < 4) {
    std::fprintf(stderr, "usage: %s N eps gemma x... gamma... dy...\n", argv[0]);
    return 1;
  }
  const int N = std::atoi(argv[1]);
  const float eps = static_cast<float>(std::atof(argv[2]));
  const int flags = std::atoi(argv[3]) ? RMSNORM_GEMMA : 0;
  if (N < 1 || argc != 4 + 3 * N) {
    std::fprintf(stderr, "expected 3 * N values after N, eps, gemma\n");
    return 1;
  }
  std::vector<float> x(N), gamma(N), dy(N);
  for (int j = 0; j < N; ++j) {
    x[j] = static_cast<float>(std::atof(argv[4 + j]));
    gamma[j] = static_cast<float>(std::atof(argv[4 + N + j]));
    dy[j] = static_cast<float>(std::atof(argv[4 + 2 * N + j]));
  }
  const int64_t M = 1;
  size_t ws_bytes = 0;
  int st = rmsnorm_bwd_workspace_bytes(M, N, RMSNORM_F32, &ws_bytes);
  if (st != RMSNORM_OK) return 3;

  float *dx_ = nullptr, *dy_ = nullptr, *x_ = nullptr, *g_ = nullptr, *y_ = nullptr, *r_ = nullptr, *dg_ = nullptr;
  void* ws = nullptr;
  CHECK_HIP(hipMalloc(&x_, N * sizeof(float)));
  CHECK_HIP(hipMalloc(&g_, N * sizeof(float)));
  CHECK_HIP(hipMalloc(&dy_, N * sizeof(float)));
  CHECK_HIP(hipMalloc(&dx_, N * sizeof(float)));
  CHECK_HIP(hipMalloc(&y_, N * sizeof(float)));
  CHECK_HIP(hipMalloc(&r_, sizeof(float)));
  CHECK_HIP(hipMalloc(&dg_, N * sizeof(float)));
  CHECK_HIP(hipMalloc(&ws, ws_bytes));
  CHECK_HIP(hipMemcpy(x_, x.data(), N * sizeof(float), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(g_, gamma.data(), N * sizeof(float), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dy_, dy.data(), N * sizeof(float), hipMemcpyHostToDevice));

  // a contract violation is a status, and nothing is launched
  st = rmsnorm_fwd(nullptr, g_, y_, r_, M, N, N, eps, RMSNORM_F32, flags, nullptr);
  if (st != RMSNORM_E_NULL) {
    std::fprintf(stderr, "null x gave status %d (%s)\n", st, rmsnorm_status_string(st));
    return 4;
  }
  std::printf("rejected %d %s\n", st, rmsnorm_status_string(st));

  st = rmsnorm_fwd(x_, g_, y_, r_, M, N, N, eps, RMSNORM_F32, flags, nullptr);
  if (st != RMSNORM_OK) return 5;
  st = rmsnorm_bwd(x_, g_, dy_, r_, dx_, dg_, ws, ws_bytes, M, N, N, RMSNORM_F32, flags, nullptr);
  if (st != RMSNORM_OK) return 6;
  CHECK_HIP(hipDeviceSynchronize());

  std::vector<float> y(N), r(1), dx(N), dg(N);
  CHECK_HIP(hipMemcpy(y.data(), y_, N * sizeof(float), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(r.data(), r_, sizeof(float), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(dx.data(), dx_, N * sizeof(float), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(dg.data(), dg_, N * sizeof(float), hipMemcpyDeviceToHost));
  print_row("y", y);
  print_row("r", r);
  print_row("dx", dx);
  print_row("dgamma", dg);
  for (void* p : {static_cast<void*>(x_), static_cast<void*>(g_), static_cast<void*>(dy_), static_cast<void*>(dx_),
                  static_cast<void*>(y_), static_cast<void*>(r_), static_cast<void*>(dg_), ws})
    CHECK_HIP(hipFree(p));
  return 0;
}
