// Exhaustive host-side check of the launch planner (csrc/host_plan.h) for
// every row operation, dtype, vector width and N in [1, RMSNORM_N_MAX], at
// three row counts: a plan always exists, covers every column and row, keeps
// a lane's row data within the register model, fits a 1024-thread workgroup,
// and keeps the LDS combine buffer within 64 KB.  Built and run by
// tests/test_plan.py; prints one summary line and exits non-zero on failure.
#include <cstdio>

#include "host_plan.h"

using namespace rmsn;

int main() {
  long bad = 0, n = 0;
  const RowOp ops[4] = {RowOp::kRmsFwd, RowOp::kRmsBwd, RowOp::kLnFwd, RowOp::kLnBwd};
  for (int dt = 0; dt < 3; ++dt)
    for (RowOp op : ops)
      for (int64_t N = 1; N <= RMSNORM_N_MAX; ++N)
        for (int vec = 1; vec <= 16 / elsize(dt); vec *= 2) {
          if (N % vec) continue;
          const bool bwd = op == RowOp::kRmsBwd || op == RowOp::kLnBwd;
          for (int64_t M : {int64_t(1), int64_t(4096), int64_t(1) << 20}) {
            const RowPlan p = plan_rows(M, N, vec, elsize(dt), lane_elems_cap(op, elsize(dt)), bwd);
            ++n;
            const int64_t lds = p.rpb > 1 ? (op == RowOp::kLnBwd ? 8 : 4) * N : 0;
            const bool ok = p.iters > 0 && p.vec * p.iters <= lane_elems_cap(op, elsize(dt)) && p.threads() <= 1024 &&
                            int64_t(p.iters) * kWave * p.wpr * vec >= N && lds <= 65536 &&
                            p.grid * p.row_iters * p.rpb >= M && (!bwd || p.grid <= kBwdGridMax);
            if (!ok && bad++ < 10)
              std::printf("bad plan: dtype=%d op=%d N=%ld vec=%d M=%ld iters=%d wpr=%d rpb=%d grid=%ld\n", dt,
                          static_cast<int>(op), static_cast<long>(N), vec, static_cast<long>(M), p.iters, p.wpr, p.rpb,
                          static_cast<long>(p.grid));
          }
        }
  std::printf("checked %ld plans, %ld bad\n", n, bad);
  return bad ? 1 : 0;
}
