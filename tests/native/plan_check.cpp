// Exhaustive host-side check of the launch planner (csrc/host_plan.h) for
// every row operation, dtype, vector width and N in [1, RMSNORM_N_MAX], at
// three row counts: a plan always exists, covers every column and row, keeps
// a lane's row data within the register model, fits a 1024-thread workgroup,
// keeps the LDS combine buffer within 64 KB, and gives no row a wave that
// lies wholly past N.  It also pins the row shapes
// the planner picks for a few widths where the ordering of its rules
// matters.  For 16-bit LayerNorm rows beyond RMSNORM_N_MAX (up to
// LAYERNORM_N_MAX_16BIT) it checks that the wide plan covers the row within
// the wide kernels' registers, and that the backward over 16-byte vectors
// gets a chunk count its held-row kernel is compiled for.  It pins the
// grids the grid rules pick at a few shapes as well.  Built and
// run by tests/test_plan.py; prints one summary line and exits non-zero on
// failure.
#include <cstdio>

#include "host_plan.h"
#include "launch.h"
#include "layernorm.h"

#include <cstring>
#include <map>
#include <set>
#include <tuple>

using namespace rmsn;

static bool in_iters_set(int it) {
  for (int v : kItersSet)
    if (v == it) return true;
  return false;
}

// With --widths: for every distinct plan (operation, element size, vector
// width, waves per row, vectors per lane) over N <= RMSNORM_N_MAX, the
// smallest and the largest N that get it, as lines "rms|ln <element size> N"
// (each norm's forward and backward both run at every width listed for it).
// The GPU test tests/test_plan_coverage_gpu.py runs each line against the
// oracle, so every row shape the planner can emit runs at least once.
static int print_widths() {
  std::map<std::tuple<int, int, int, int, int>, std::pair<int64_t, int64_t>> first_last;
  const RowOp ops[4] = {RowOp::kRmsFwd, RowOp::kRmsBwd, RowOp::kLnFwd, RowOp::kLnBwd};
  for (int es : {2, 4})
    for (RowOp op : ops)
      for (int vec = 16 / es; vec >= 1; vec /= 2)
        for (int64_t N = vec; N <= RMSNORM_N_MAX; N += vec) {
          if (vec < 16 / es && N % (2 * vec) == 0) continue;  // N alone would allow a wider vector
          const RowPlan p = plan_rows(op, 33, N, vec, es == 4 ? 0 : 1);
          const auto key = std::make_tuple(static_cast<int>(op), es, vec, p.wpr, p.iters);
          auto it = first_last.find(key);
          if (it == first_last.end())
            first_last[key] = {N, N};
          else
            it->second.second = N;
        }
  std::set<std::tuple<int, int, int64_t>> widths;  // (LayerNorm?, element size, N)
  for (const auto& [key, range] : first_last) {
    const int ln = std::get<0>(key) >= static_cast<int>(RowOp::kLnFwd);
    widths.insert({ln, std::get<1>(key), range.first});
    widths.insert({ln, std::get<1>(key), range.second});
  }
  for (const auto& [ln, es, N] : widths) std::printf("%s %d %ld\n", ln ? "ln" : "rms", es, static_cast<long>(N));
  return 0;
}

int main(int argc, char** argv) {
  if (argc > 1 && std::strcmp(argv[1], "--widths") == 0) return print_widths();
  long bad = 0, n = 0;
  const RowOp ops[4] = {RowOp::kRmsFwd, RowOp::kRmsBwd, RowOp::kLnFwd, RowOp::kLnBwd};
  for (int dt = 0; dt < 3; ++dt)
    for (RowOp op : ops)
      for (int64_t N = 1; N <= RMSNORM_N_MAX; ++N)
        for (int vec = 1; vec <= 16 / elsize(dt); vec *= 2) {
          if (N % vec) continue;
          const bool bwd = op == RowOp::kRmsBwd || op == RowOp::kLnBwd;
          for (int64_t M : {int64_t(1), int64_t(4096), int64_t(1) << 20}) {
            const RowPlan p = plan_rows(op, M, N, vec, dt);
            ++n;
            const int64_t lds = p.rpb > 1 ? (op == RowOp::kLnBwd ? 8 : 4) * N : 0;
            const bool ok = p.iters > 0 && p.vec * p.iters <= lane_elems_cap(op, elsize(dt)) && p.threads() <= 1024 &&
                            int64_t(p.iters) * kWave * p.wpr * vec >= N && lds <= 65536 &&
                            p.grid * p.row_iters * p.rpb >= M && (!bwd || p.grid <= kBwdGridMax) &&
                            // no wave of a row lies wholly past N (in either lane mapping)
                            (p.wpr == 1 || int64_t(p.wpr - 1) * p.iters * kWave < N / vec);
            if (!ok && bad++ < 10)
              std::printf("bad plan: dtype=%d op=%d N=%ld vec=%d M=%ld iters=%d wpr=%d rpb=%d grid=%ld\n", dt,
                          static_cast<int>(op), static_cast<long>(N), vec, static_cast<long>(M), p.iters, p.wpr, p.rpb,
                          static_cast<long>(p.grid));
          }
        }
  // 16-bit LayerNorm rows beyond the register plans: the wide kernels
  static_assert(kLnWideMaxN == LAYERNORM_N_MAX_16BIT, "wide kernels cover every LayerNorm row");
  for (int dt = 1; dt < 3; ++dt)
    for (bool bwd : {false, true})
      for (int64_t N = RMSNORM_N_MAX + 1; N <= LAYERNORM_N_MAX_16BIT; ++N)
        for (int vec = 1; vec <= 8; vec *= 2) {
          if (N % vec) continue;
          for (int64_t M : {int64_t(1), int64_t(300), int64_t(1) << 20}) {
            ++n;
            const RowPlan p = plan_ln_wide(bwd, M, N, vec);
            const bool ok = p.vec == vec && p.wpr * kWave == 1024 && p.rpb == 1 && p.iters >= 1 &&
                            int64_t(p.iters) * 1024 * vec >= N && p.iters * vec <= kLnWideColsPerLane &&
                            p.grid >= 1 && p.grid * p.row_iters >= M && (!bwd || p.grid <= wide_partial_rows_bound(M)) &&
                            // the backward over 16-byte vectors: a compiled held-row chunk count
                            (!bwd || vec * 2 != 16 ||
                             (p.iters >= kLnWideHeldChunksMin && p.iters <= kLnWideHeldChunksMax &&
                              kLnWideHeldLdsBytes(p.iters) + 256 <= kLdsPerWorkgroup));
            if (!ok && bad++ < 10)
              std::printf("bad wide plan: dtype=%d bwd=%d N=%ld vec=%d M=%ld chunks=%d grid=%ld\n", dt, int(bwd),
                          static_cast<long>(N), vec, static_cast<long>(M), p.iters, static_cast<long>(p.grid));
          }
        }
  // the LayerNorm forward of those rows: a register plan of at most
  // kLnWideRegWaves (16-byte vectors) / kLnWideRegWavesNarrow waves, else wide
  long fwd_reg = 0, fwd_wide = 0;
  for (int dt = 1; dt < 3; ++dt)
    for (int64_t N = RMSNORM_N_MAX + 1; N <= LAYERNORM_N_MAX_16BIT; ++N)
      for (int vec = 1; vec <= 8; vec *= 2) {
        if (N % vec) continue;
        for (int64_t M : {int64_t(1), int64_t(4096), int64_t(1) << 20}) {
          ++n;
          const RowPlan p = plan_ln_fwd(M, N, vec, dt);
          bool ok;
          if (p.wide) {
            ++fwd_wide;
            ok = p.vec == vec && p.wpr * kWave == 1024 && p.rpb == 1 && int64_t(p.iters) * 1024 * vec >= N &&
                 p.iters * vec <= kLnWideColsPerLane && p.grid * p.row_iters >= M;
          } else {
            ++fwd_reg;
            const int max_waves = vec * 2 == 16 ? kLnWideRegWaves : kLnWideRegWavesNarrow;
            ok = in_iters_set(p.iters) && p.vec * p.iters <= lane_elems_cap(RowOp::kLnFwd, 2) && p.wpr <= max_waves &&
                 p.threads() <= 1024 && int64_t(p.iters) * kWave * p.wpr * vec >= N &&
                 p.grid * p.row_iters * p.rpb >= M && (p.wpr == 1 || int64_t(p.wpr - 1) * p.iters * kWave < N / vec);
          }
          if (!ok && bad++ < 10)
            std::printf("bad wide forward plan: dtype=%d N=%ld vec=%d M=%ld wide=%d iters=%d wpr=%d\n", dt,
                        static_cast<long>(N), vec, static_cast<long>(M), int(p.wide), p.iters, p.wpr);
        }
      }
  if (fwd_reg == 0 || fwd_wide == 0) {
    ++bad;
    std::printf("wide forward: %ld register plans, %ld wide plans\n", fwd_reg, fwd_wide);
  }
  // (element size, N, op, waves per row, vectors per lane), 16-byte vectors
  struct Pin {
    int es;
    int64_t N;
    RowOp op;
    int wpr, iters;
  };
  const Pin pins[] = {
      {2, 8192, RowOp::kRmsFwd, 8, 2},   {2, 8192, RowOp::kRmsBwd, 8, 2},    // no waste
      {2, 7680, RowOp::kRmsFwd, 8, 2},   {2, 7680, RowOp::kLnBwd, 8, 2},     // not 15 x 1
      {2, 2560, RowOp::kLnFwd, 1, 5},    {2, 4608, RowOp::kRmsBwd, 5, 2},    // forward: not 3 x 2; not 5 x 1, 9 x 1
      {2, 3072, RowOp::kLnFwd, 3, 2},    {2, 2560, RowOp::kLnBwd, 3, 2},     // three waves kept
      {2, 16384, RowOp::kRmsFwd, 8, 4},  {2, 16384, RowOp::kRmsBwd, 16, 2},  // forward rows of <= 8 waves
      {2, 13312, RowOp::kLnFwd, 7, 4},   {2, 13312, RowOp::kLnBwd, 13, 2},
      {2, 1536, RowOp::kRmsFwd, 1, 4},   {2, 1536, RowOp::kRmsBwd, 2, 2},    // not 3 x 1
      {2, 1232, RowOp::kLnFwd, 1, 4},    {2, 2048, RowOp::kRmsFwd, 2, 2},    // one wave; 2 x 2 where exact
      {2, 3200, RowOp::kRmsFwd, 4, 2},   {2, 3200, RowOp::kLnBwd, 4, 2},     // not 7 x 1
      {2, 2304, RowOp::kRmsBwd, 3, 2},   {4, 704, RowOp::kRmsFwd, 2, 2},     // not 5 x 1, 3 x 1
      {4, 1100, RowOp::kLnBwd, 3, 2},    {4, 1600, RowOp::kRmsBwd, 4, 2},    // not 5 x 1, 7 x 1
      {4, 1200, RowOp::kRmsBwd, 3, 2},                                        // not 1 x 5
      {2, 9216, RowOp::kLnFwd, 4, 5},    {2, 10240, RowOp::kLnFwd, 5, 4},    // LayerNorm forward
      {2, 9216, RowOp::kRmsFwd, 5, 4},   {2, 5264, RowOp::kLnFwd, 3, 4},
      {2, 6432, RowOp::kLnFwd, 4, 4},    {2, 6432, RowOp::kRmsFwd, 7, 2},
      {4, 14848, RowOp::kRmsFwd, 12, 5}, {4, 7680, RowOp::kRmsFwd, 6, 5},    // fp32: least waste first
      {4, 3328, RowOp::kRmsFwd, 7, 2},                                        // not 13 x 1
  };
  for (const Pin& q : pins) {
    const RowPlan p = plan_rows(q.op, 4096, q.N, 16 / q.es, q.es == 4 ? 0 : 1);
    ++n;
    if (p.wpr != q.wpr || p.iters != q.iters) {
      ++bad;
      std::printf("shape pin: es=%d N=%ld op=%d: got %d x %d, expected %d x %d\n", q.es, static_cast<long>(q.N),
                  static_cast<int>(q.op), p.wpr, p.iters, q.wpr, q.iters);
    }
  }
  // grids the planner's rules pick, 16-byte vectors: (element size, M, N,
  // op, dtype, workgroups, row groups per workgroup, row steps, and 1 / 0:
  // the backward pipelined, the RMSNorm forward's first row loaded early;
  // -1 for the LayerNorm forward)
  struct GridPin {
    int es;
    int64_t M, N;
    RowOp op;
    int dtype;
    int64_t grid;
    int rpb;
    int64_t row_iters;
    int pipelined;
  };
  const GridPin grid_pins[] = {
      // backward: one pipelined workgroup of the row's shape per CU wherever
      // the pipelined loop is compiled
      {2, 16384, 8192, RowOp::kRmsBwd, 1, 256, 1, 64, 1},    // the headline
      {2, 32768, 5120, RowOp::kRmsBwd, 1, 256, 1, 128, 1},   // 5-wave rows alone on a CU
      {2, 4096, 4096, RowOp::kRmsBwd, 1, 256, 2, 8, 1},      // 4-wave rows, two row groups
      {2, 32768, 4096, RowOp::kLnBwd, 2, 256, 2, 64, 1},
      // ... 16-wave workgroups for 5-8-wave rows where the partial rows weigh
      {2, 4096, 6144, RowOp::kLnBwd, 2, 256, 2, 8, 1},
      // bf16 LayerNorm: pipelined in its build for workgroups of at most 512
      // threads, except rows of 5-8 waves where the partial rows weigh (one
      // 16-wave workgroup per CU, not pipelined)
      {2, 32768, 4096, RowOp::kLnBwd, 1, 256, 2, 64, 1},
      {2, 4096, 4096, RowOp::kLnBwd, 1, 256, 2, 8, 1},
      {2, 4096, 6144, RowOp::kLnBwd, 1, 256, 2, 8, 0},
      // forward of 3-6 row steps (LayerNorm; 3-4 RMSNorm): 1024 workgroups of
      // one row group, for rows of >= 7 KiB and <= 5 waves
      {2, 4096, 4096, RowOp::kLnFwd, 2, 1024, 1, 4, -1},
      {2, 4096, 4096, RowOp::kRmsFwd, 1, 1024, 1, 4, 1},
      {2, 6000, 5632, RowOp::kLnFwd, 2, 1024, 1, 6, -1},
      {2, 2049, 3584, RowOp::kRmsFwd, 1, 1024, 1, 3, 1},
      {2, 6000, 4096, RowOp::kRmsFwd, 1, 3000, 2, 1, 0},        // 6 steps: RMSNorm keeps the other rules
      // ... and rows of 2-7 KiB where the rows divide evenly into 2-6 steps
      // (2-4 RMSNorm) over a whole number of workgroups per CU, at most four
      {2, 4096, 3072, RowOp::kLnFwd, 2, 1024, 2, 2, -1},     // 3-wave rows, two per workgroup
      {2, 4096, 3328, RowOp::kRmsFwd, 1, 1024, 2, 2, 1},        // 4-wave rows
      {2, 12288, 2816, RowOp::kLnFwd, 2, 1024, 2, 6, -1},
      {2, 12288, 2816, RowOp::kRmsFwd, 1, 6144, 2, 1, 0},       // 6 steps: RMSNorm keeps the other rules
      {2, 6144, 2304, RowOp::kLnFwd, 2, 768, 4, 2, -1},      // 1-wave rows, four per workgroup
      {2, 16384, 2048, RowOp::kRmsFwd, 1, 1024, 4, 4, 1},       // 2-wave rows
      {2, 5000, 3072, RowOp::kLnFwd, 2, 2500, 2, 1, -1},     // rows that do not divide evenly
      {2, 8192, 1024, RowOp::kLnFwd, 2, 1024, 8, 1, -1},     // 2 KiB rows
      // the RMSNorm forward's first row loaded early: persistent grids and
      // grids of at most 2048 workgroups, not large one-step grids
      {2, 16384, 8192, RowOp::kRmsFwd, 1, 512, 1, 32, 1},    // the headline
      {2, 4096, 2048, RowOp::kRmsFwd, 1, 1024, 4, 1, 1},
      {2, 32768, 5120, RowOp::kRmsFwd, 1, 32768, 1, 1, 0},
      {2, 4096, 12288, RowOp::kLnFwd, 2, 512, 1, 8, -1},     // 6-wave rows of four vectors: persistent, two per CU
      {2, 2048, 6144, RowOp::kLnFwd, 2, 1024, 2, 1, -1},     // 2 steps: one workgroup per two 3 x 4 row groups
  };
  for (const GridPin& q : grid_pins) {
    const RowPlan p = plan_rows(q.op, q.M, q.N, 16 / q.es, q.dtype);
    ++n;
    const int pipe = q.op == RowOp::kRmsBwd || q.op == RowOp::kLnBwd ? int(bwd_pipelined(q.op, p, q.dtype))
                     : q.op == RowOp::kRmsFwd                          ? int(fwd_first_row_early(p))
                                                                       : -1;
    if (p.grid != q.grid || p.rpb != q.rpb || p.row_iters != q.row_iters || pipe != q.pipelined) {
      ++bad;
      std::printf("grid pin: op=%d dtype=%d %ld x %ld: got grid %ld, %d row groups, %ld steps, pipelined %d; expected "
                  "%ld, %d, %ld, %d\n",
                  static_cast<int>(q.op), q.dtype, static_cast<long>(q.M), static_cast<long>(q.N),
                  static_cast<long>(p.grid), p.rpb, static_cast<long>(p.row_iters), pipe, static_cast<long>(q.grid),
                  q.rpb, static_cast<long>(q.row_iters), q.pipelined);
    }
  }
  std::printf("checked %ld plans, %ld bad\n", n, bad);
  return bad ? 1 : 0;
}
