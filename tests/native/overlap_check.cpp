// Brute-force check of matrices_overlap (csrc/host_plan.h): for small shapes,
// strides, element sizes and byte offsets, the exact answer (do the two sets
// of row-segment bytes intersect?) against the function.  Built and run by
// tests/test_plan.py; exits non-zero on a mismatch.
#include <cstdio>
#include <set>

#include "host_plan.h"

using namespace rmsn;

int main() {
  long checked = 0, bad = 0;
  for (int es : {1, 2, 4})
    for (int64_t M = 1; M <= 4; ++M)
      for (int64_t N = 1; N <= 5; ++N)
        for (int64_t S = N; S <= N + 6; ++S)
          for (int64_t d = -40; d <= 40; ++d) {
            std::set<int64_t> a;
            for (int64_t r = 0; r < M; ++r)
              for (int64_t c = 0; c < N * es; ++c) a.insert(r * S * es + c);
            bool want = false;
            for (int64_t r = 0; r < M && !want; ++r)
              for (int64_t c = 0; c < N * es; ++c)
                if (a.count(d + r * S * es + c)) {
                  want = true;
                  break;
                }
            const char* base = reinterpret_cast<const char*>(0x100000);
            const bool got = matrices_overlap(base, base + d, M, N, S, es);
            ++checked;
            if (got != want && bad++ < 10)
              std::printf("mismatch es=%d M=%ld N=%ld S=%ld d=%ld: got %d want %d\n", es, static_cast<long>(M),
                          static_cast<long>(N), static_cast<long>(S), static_cast<long>(d), got, want);
          }
  std::printf("checked %ld cases, %ld bad\n", checked, bad);
  return bad ? 1 : 0;
}
