// The host side of every entry point, built without any device code: the
// launchers are replaced by stubs that check what the host hands the kernels
// (launch plan, kernel arguments, descriptor ranges, LDS size, grid limits)
// and launch nothing.  The driver calls every entry point over a grid of
// shapes, dtypes, row strides, flags, in-place and misaligned cases with
// valid (never dereferenced) device addresses: each such call must return
// RMSNORM_OK and hand the kernels a consistent plan.  Built and run by
// tests/test_host_contract.py with AddressSanitizer and UndefinedBehavior-
// Sanitizer, which also watch the validation arithmetic itself.  Prints one
// summary line and exits non-zero on any failure.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <limits>
#include <initializer_list>

#include "host_plan.h"
#include "launch.h"
#include "layernorm.h"
#include "rmsnorm.h"
#include "rope.h"
#include "swiglu.h"

namespace {
long g_checks = 0, g_bad = 0, g_launches = 0;

void expect(bool ok, const char* what, long long a = 0, long long b = 0) {
  ++g_checks;
  if (!ok && g_bad++ < 20) std::printf("failed: %s (%lld, %lld)\n", what, a, b);
}

int elsize_of(int dtype) { return dtype == 0 ? 4 : 2; }
bool in_iters_set(int it) {
  for (int v : rmsn::kItersSet)
    if (v == it) return true;
  return false;
}

// What every row-kernel launch must satisfy.
void check_row_plan(const rmsn::RowPlan& p, rmsn::RowOp op, int dtype, int64_t M, int64_t stride, int32_t N,
                    int32_t nvec, int32_t wpr, int32_t rpb, int64_t row_iters) {
  using namespace rmsn;
  const int es = elsize_of(dtype);
  const bool bwd = op == RowOp::kRmsBwd || op == RowOp::kLnBwd;
  expect(p.vec == 1 || p.vec == 2 || p.vec == 4 || p.vec == 8, "vector width", p.vec);
  expect(p.vec * es <= 16, "vector bytes", p.vec * es);
  expect(N % p.vec == 0 && stride % p.vec == 0, "width divides N and the stride", N, stride);
  expect(int64_t(nvec) * p.vec == N, "nvec * vec == N", nvec, N);
  expect(in_iters_set(p.iters), "iters compiled", p.iters);
  expect(p.vec * p.iters <= lane_elems_cap(op, es), "register model", p.vec * p.iters);
  expect(p.wpr >= 1 && p.wpr <= kMaxBlockWaves && p.rpb >= 1 && p.threads() <= 1024, "workgroup shape", p.wpr,
         p.rpb);
  expect(int64_t(p.iters) * kWave * p.wpr * p.vec >= N, "row covered", N);
  expect(p.grid >= 1 && p.grid <= (int64_t(1) << 31) - 1, "grid size", p.grid);
  expect(p.grid * p.row_iters * p.rpb >= M, "rows covered", M);
  expect(!bwd || p.grid <= kBwdGridMax, "backward grid", p.grid);
  expect(wpr == p.wpr && rpb == p.rpb && row_iters == p.row_iters, "arguments match the plan");
  expect(stride >= N, "stride", stride, N);
  expect(int64_t(N) * es < (int64_t(1) << 31), "row descriptor range", N);
  expect(M * 4 <= (int64_t(1) << 31), "per-row scalar descriptor range", M);
}
}  // namespace

namespace rmsn {
// The static scratch of rmsnorm_bwd_noalloc, stood in for by a fake address.
char* const kScratch = reinterpret_cast<char*>(uintptr_t(1) << 45);
long g_scratch_lookups = 0;
hipError_t static_scratch(void** ptr) {
  ++g_scratch_lookups;
  *ptr = kScratch;
  return hipSuccess;
}
hipError_t launch_fwd(int dtype, const RowPlan& p, const FwdArgs& a, hipStream_t) {
  ++g_launches;
  check_row_plan(p, RowOp::kRmsFwd, dtype, a.M, a.stride, a.N, a.nvec, a.wpr, a.rpb, a.row_iters);
  expect(a.x && a.gamma && a.y && a.rstd, "forward pointers");
  return hipSuccess;
}
hipError_t launch_bwd_rows(int dtype, const RowPlan& p, const BwdArgs& a, hipStream_t) {
  ++g_launches;
  check_row_plan(p, RowOp::kRmsBwd, dtype, a.M, a.stride, a.N, a.nvec, a.wpr, a.rpb, a.row_iters);
  expect(p.rpb == 1 || int64_t(a.N) * 4 <= 65536, "LDS combine size", a.N);
  expect(!a.pipeline || (bwd_pipeline_fits(RowOp::kRmsBwd, dtype, p.vec, p.iters, p.threads()) &&
                         (p.wpr * p.rpb * 2 > kBwdResidentWaves || p.grid <= kComputeUnits)),
         "pipelined only where it fits and the workgroup is alone on its CU");
  expect(p.grid <= partial_rows_bound(a.M), "partial rows within the workspace", p.grid);
  expect(a.partials_nt == int(partials_nontemporal(1, p.grid, a.N)), "partial-row store policy", p.grid, a.N);
  expect(reinterpret_cast<const char*>(a.partials) != kScratch ||
             p.grid * int64_t(a.N) * 4 <= RMSNORM_STATIC_SCRATCH_BYTES,
         "partial rows within the static scratch", p.grid, a.N);
  return hipSuccess;
}
hipError_t launch_dgamma_reduce(int vec, int tables, const ReduceArgs& a, hipStream_t) {
  ++g_launches;
  expect(vec == 1 || vec == 4, "reduce width", vec);
  expect(tables == 1 || tables == 2, "tables", tables);
  expect((tables == 2) == (a.dgamma2 != nullptr), "second output iff two tables");
  expect(a.rows >= 0 && a.rows * a.N * 4 <= (int64_t(1) << 31), "partials descriptor range", a.rows, a.N);
  expect(a.N % vec == 0, "reduce width divides N", a.N, vec);
  return hipSuccess;
}
hipError_t launch_ln_fwd(int dtype, const RowPlan& p, const LnFwdArgs& a, hipStream_t) {
  ++g_launches;
  check_row_plan(p, RowOp::kLnFwd, dtype, a.M, a.stride, a.N, a.nvec, a.wpr, a.rpb, a.row_iters);
  return hipSuccess;
}
hipError_t launch_ln_bwd_rows(int dtype, const RowPlan& p, const LnBwdArgs& a, hipStream_t) {
  ++g_launches;
  check_row_plan(p, RowOp::kLnBwd, dtype, a.M, a.stride, a.N, a.nvec, a.wpr, a.rpb, a.row_iters);
  expect(p.rpb == 1 || int64_t(a.N) * 8 <= 65536, "LDS combine size", a.N);
  expect(a.partials_nt == int(partials_nontemporal(2, p.grid, a.N)), "partial-row store policy", p.grid, a.N);
  expect(!a.pipeline || (bwd_pipeline_fits(RowOp::kLnBwd, dtype, p.vec, p.iters, p.threads()) &&
                         (p.wpr * p.rpb * 2 > kBwdResidentWaves || p.grid <= kComputeUnits)),
         "pipelined only where it fits and the workgroup is alone on its CU");
  return hipSuccess;
}
// What every wide LayerNorm launch must satisfy (16-bit rows beyond the
// register plans, one 1024-thread workgroup per row).
static void check_wide_plan(const RowPlan& p, bool bwd, int dtype, int64_t M, int64_t stride, int32_t N, int32_t nvec,
                            int32_t chunks, int64_t row_iters) {
  expect(dtype == 1 || dtype == 2, "wide rows are 16-bit", dtype);
  expect(N > RMSNORM_N_MAX && N <= kLnWideMaxN, "wide rows only beyond the register plans", N);
  expect(p.vec == 1 || p.vec == 2 || p.vec == 4 || p.vec == 8, "wide vector width", p.vec);
  expect(N % p.vec == 0 && stride % p.vec == 0 && int64_t(nvec) * p.vec == N, "wide width divides N", N, stride);
  expect(p.wpr * kWave == 1024 && p.rpb == 1, "wide workgroup", p.wpr, p.rpb);
  expect(chunks == p.iters && int64_t(chunks) * 1024 >= nvec, "wide row covered", chunks, nvec);
  expect(chunks * p.vec <= kLnWideColsPerLane, "wide columns per lane", chunks, p.vec);
  expect(p.grid >= 1 && p.grid * row_iters >= M && row_iters == p.row_iters, "wide rows covered", M);
  expect(!bwd || p.grid <= wide_partial_rows_bound(M), "wide partial rows within the workspace", p.grid);
  expect(int64_t(N) * 2 < (int64_t(1) << 31) && M * 4 <= (int64_t(1) << 31), "wide descriptor ranges", N, M);
}
long g_wide_launches = 0;
hipError_t launch_ln_fwd_wide(int dtype, const RowPlan& p, const LnFwdArgs& a, hipStream_t) {
  ++g_launches;
  ++g_wide_launches;
  check_wide_plan(p, false, dtype, a.M, a.stride, a.N, a.nvec, a.chunks, a.row_iters);
  return hipSuccess;
}
hipError_t launch_ln_bwd_wide(int dtype, const RowPlan& p, const LnBwdArgs& a, hipStream_t) {
  ++g_launches;
  ++g_wide_launches;
  check_wide_plan(p, true, dtype, a.M, a.stride, a.N, a.nvec, a.chunks, a.row_iters);
  expect(!a.pipeline, "wide backward not pipelined");
  expect(!a.partials_nt, "wide partial rows with the default policy");
  return hipSuccess;
}
hipError_t launch_rope(int dtype, int vec, const RopeArgs& a, hipStream_t) {
  ++g_launches;
  const int es = elsize_of(dtype);
  expect(vec >= 1 && vec * es <= 16 && a.half % vec == 0, "rope width", vec, a.half);
  expect(a.nvh * vec == a.half, "rope vectors per half");
  expect(a.groups == (a.heads + kRopeGroup - 1) / kRopeGroup, "rope head groups");
  expect(a.items == a.tokens * a.groups * a.nvh, "rope items");
  expect((a.items + kEltThreads - 1) / kEltThreads * kEltThreads <= (int64_t(1) << 32) - 1,
         "rope work items fit a dispatch");
  expect(a.table_rows * a.half * 4 < (int64_t(1) << 31), "table descriptor range");
  expect(int64_t(a.heads) * a.half * 2 * es < (int64_t(1) << 31), "token descriptor range");
  expect(a.sin_sign == 1.0f || a.sin_sign == -1.0f, "rope direction");
  return hipSuccess;
}
static void check_swiglu(int dtype, int vec, const SwigluArgs& a) {
  const int es = elsize_of(dtype);
  expect(vec >= 1 && vec * es <= 16 && a.N % vec == 0, "swiglu width", vec, a.N);
  expect(a.tiles == (a.N / vec + kSwigluUnroll * kEltThreads - 1) / (kSwigluUnroll * kEltThreads), "swiglu tiles");
  expect(a.blocks == a.M * a.tiles, "swiglu blocks");
  expect(a.last_row_elems >= 1 && a.last_row_elems <= a.N, "last row length", a.last_row_elems, a.N);
  expect(a.stride >= a.N && int64_t(a.N) * es < (int64_t(1) << 31), "swiglu row range", a.N);
}
hipError_t launch_swiglu_fwd(int dtype, int vec, const SwigluArgs& a, hipStream_t) {
  ++g_launches;
  check_swiglu(dtype, vec, a);
  return hipSuccess;
}
hipError_t launch_swiglu_bwd(int dtype, int vec, const SwigluArgs& a, hipStream_t) {
  ++g_launches;
  check_swiglu(dtype, vec, a);
  expect(a.dh && a.df && a.de, "backward pointers");
  return hipSuccess;
}
}  // namespace rmsn

namespace {
// Far-apart, 256-byte aligned device addresses (never dereferenced): slot k
// lies at k * 2^46 bytes, more than any matrix the ABI accepts spans.
char* slot(int k, int64_t misalign_bytes = 0) {
  return reinterpret_cast<char*>((uintptr_t(1) << 46) * uintptr_t(k + 1) + uintptr_t(misalign_bytes));
}

void expect_ok(int st, const char* what, int64_t M, int64_t N) {
  expect(st == RMSNORM_OK, what, M, N);
  if (st != RMSNORM_OK && g_bad <= 20) std::printf("   status %d: %s\n", st, rmsnorm_status_string(st));
}

void layernorms(int64_t M, int64_t N, int64_t stride, int dtype, int64_t off);

void norms(int64_t M, int64_t N, int64_t stride, int dtype, int64_t mis) {
  const int es = elsize_of(dtype);
  const int64_t off = mis * es;  // element-aligned, possibly not 16-byte aligned
  size_t wbytes = 0;
  expect_ok(rmsnorm_bwd_workspace_bytes(M, N, dtype, &wbytes), "rms workspace query", M, N);
  const hipStream_t s = nullptr;
  for (int flags : {0, int(RMSNORM_GEMMA), int(RMSNORM_GEMMA | RMSNORM_ROUND_NORMED)}) {
    expect_ok(rmsnorm_fwd(slot(0, off), slot(1), slot(2, off), reinterpret_cast<float*>(slot(3)), M, N, stride, 1e-6f,
                          dtype, flags, s),
              "rmsnorm_fwd", M, N);
    for (bool in_place : {false, true}) {
      void* dy = slot(4, off);
      void* dx = in_place ? dy : slot(5, off);
      int64_t rows = -1;
      expect_ok(rmsnorm_bwd_rows(slot(0, off), slot(1), dy, reinterpret_cast<const float*>(slot(3)), dx, slot(6),
                                 wbytes, M, N, stride, dtype, flags & RMSNORM_GEMMA, &rows, s),
                "rmsnorm_bwd_rows", M, N);
      expect(rows >= 0 && rows <= rmsn::partial_rows_bound(M), "partial rows reported", rows, M);
      expect_ok(rmsnorm_bwd(slot(0, off), slot(1), dy, reinterpret_cast<const float*>(slot(3)), dx,
                            reinterpret_cast<float*>(slot(7)), slot(6), wbytes, M, N, stride, dtype,
                            flags & RMSNORM_GEMMA, s),
                "rmsnorm_bwd", M, N);
      expect_ok(rmsnorm_bwd_noalloc(slot(0, off), slot(1), dy, reinterpret_cast<const float*>(slot(3)), dx,
                                    reinterpret_cast<float*>(slot(7)), M, N, stride, dtype, flags & RMSNORM_GEMMA, s),
                "rmsnorm_bwd_noalloc", M, N);
    }
  }
  layernorms(M, N, stride, dtype, off);
}

void layernorms(int64_t M, int64_t N, int64_t stride, int dtype, int64_t off) {
  size_t lwbytes = 0;
  expect_ok(layernorm_bwd_workspace_bytes(M, N, dtype, &lwbytes), "ln workspace query", M, N);
  const hipStream_t s = nullptr;
  expect_ok(layernorm_fwd(slot(0, off), slot(1), slot(8), slot(2, off), reinterpret_cast<float*>(slot(3)),
                          reinterpret_cast<float*>(slot(9)), M, N, stride, 1e-5f, dtype, s),
            "layernorm_fwd", M, N);
  for (bool in_place : {false, true}) {
    void* dy = slot(4, off);
    void* dx = in_place ? dy : slot(5, off);
    int64_t rows = -1;
    expect_ok(layernorm_bwd_rows(slot(0, off), slot(1), dy, reinterpret_cast<const float*>(slot(3)),
                                 reinterpret_cast<const float*>(slot(9)), dx, slot(6), lwbytes, M, N, stride, dtype,
                                 &rows, s),
              "layernorm_bwd_rows", M, N);
    expect_ok(layernorm_bwd(slot(0, off), slot(1), dy, reinterpret_cast<const float*>(slot(3)),
                            reinterpret_cast<const float*>(slot(9)), dx, reinterpret_cast<float*>(slot(7)),
                            reinterpret_cast<float*>(slot(10)), slot(6), lwbytes, M, N, stride, dtype, s),
              "layernorm_bwd", M, N);
  }
}
}  // namespace

int main() {
  const int64_t Ms[] = {0, 1, 7, 17, 300, 4096, 16384, 65537, int64_t(1) << 20, int64_t(1) << 29};
  const int64_t Ns[] = {1, 2, 3, 8, 96, 257, 1000, 1024, 1536, 2560, 4096, 5120, 7680, 8192, 9216, 13312, 15872,
                        16383, 16384};
  for (int dtype = 0; dtype < 3; ++dtype)
    for (int64_t M : Ms)
      for (int64_t N : Ns)
        for (int64_t pad : {0, 1, 8, 64})
          for (int64_t mis : {0, 1}) norms(M, N, N + pad, dtype, mis);

  // 16-bit LayerNorm rows beyond RMSNORM_N_MAX run in the wide kernels; fp32
  // rows that long, and any row beyond LAYERNORM_N_MAX_16BIT, are rejected
  for (int dtype = 1; dtype < 3; ++dtype)
    for (int64_t M : {int64_t(0), int64_t(1), int64_t(255), int64_t(300), int64_t(65537), int64_t(1) << 20})
      for (int64_t N : {int64_t(16385), int64_t(16392), int64_t(20000), int64_t(24576), int64_t(32767),
                        int64_t(32768)})
        for (int64_t pad : {0, 1, 8})
          for (int64_t mis : {0, 1}) layernorms(M, N, N + pad, dtype, mis * 2);
  expect(rmsn::g_wide_launches > 0, "wide launches checked");
  {
    const long before = g_launches;
    size_t lw = 0;
    for (int64_t N : {int64_t(16385), int64_t(32768)})
      expect(layernorm_fwd(slot(0), slot(1), slot(8), slot(2), reinterpret_cast<float*>(slot(3)),
                           reinterpret_cast<float*>(slot(9)), 4, N, N, 1e-5f, 0, nullptr) == RMSNORM_E_SHAPE &&
                 layernorm_bwd_workspace_bytes(4, N, 0, &lw) == RMSNORM_E_SHAPE,
             "fp32 LayerNorm rows beyond RMSNORM_N_MAX rejected", N);
    for (int dtype = 1; dtype < 3; ++dtype)
      expect(layernorm_fwd(slot(0), slot(1), slot(8), slot(2), reinterpret_cast<float*>(slot(3)),
                           reinterpret_cast<float*>(slot(9)), 4, 32769, 32769, 1e-5f, dtype,
                           nullptr) == RMSNORM_E_SHAPE &&
                 rmsnorm_fwd(slot(0), slot(1), slot(2), reinterpret_cast<float*>(slot(3)), 4, 16385, 16385, 1e-6f,
                             dtype, 0, nullptr) == RMSNORM_E_SHAPE,
             "rows beyond each norm's limit rejected", dtype);
    expect(g_launches == before, "no launch for a rejected row length");
  }

  // RoPE: heads x head_dim per token, dense or a view of a wider (fused) row
  for (int dtype = 0; dtype < 3; ++dtype)
    for (int64_t T : {int64_t(0), int64_t(1), int64_t(33), int64_t(8192), int64_t(1) << 22})
      for (int64_t H : {1, 3, 32, 64})
        for (int64_t D : {2, 6, 64, 128, 256, 1024})
          for (int64_t extra : {int64_t(0), 2 * H * D}) {
            const int64_t stride = H * D + extra;
            // one thread per (token, group of four heads, vector of the half-head):
            // calls of more work items than a dispatch holds (2^32 - 1) are rejected
            const int64_t vec = std::min<int64_t>(16 / elsize_of(dtype), D / 2 & -(D / 2));
            const int64_t items = T * ((H + rmsn::kRopeGroup - 1) / rmsn::kRopeGroup) * (D / 2 / vec);
            if ((items + rmsn::kEltThreads - 1) / rmsn::kEltThreads * rmsn::kEltThreads > (int64_t(1) << 32) - 1) {
              const int64_t before = g_launches;
              expect(rope_fwd(slot(0), T, H, D, stride, reinterpret_cast<const float*>(slot(1)),
                              reinterpret_cast<const float*>(slot(2)), 4096, nullptr, 2048, dtype,
                              nullptr) == RMSNORM_E_SHAPE && g_launches == before,
                     "rope beyond one dispatch rejected", T, H * D);
              continue;
            }
            for (bool with_positions : {false, true}) {
              const int32_t* pos = with_positions ? reinterpret_cast<const int32_t*>(slot(3)) : nullptr;
              expect_ok(rope_fwd(slot(0), T, H, D, stride, reinterpret_cast<const float*>(slot(1)),
                                 reinterpret_cast<const float*>(slot(2)), 4096, pos, 2048, dtype, nullptr),
                        "rope_fwd", T, H * D);
              expect_ok(rope_bwd(slot(0), T, H, D, stride, reinterpret_cast<const float*>(slot(1)),
                                 reinterpret_cast<const float*>(slot(2)), 4096, pos, 2048, dtype, nullptr),
                        "rope_bwd", T, H * D);
            }
          }

  // SwiGLU: dense (walked as flat rows) and strided, outputs separate or over the inputs
  for (int dtype = 0; dtype < 3; ++dtype)
    for (int64_t M : {int64_t(0), int64_t(1), int64_t(7), int64_t(11136), int64_t(1) << 20})
      for (int64_t N : {int64_t(1), int64_t(3), int64_t(513), int64_t(14336), int64_t(70000), int64_t(1) << 26})
        for (int64_t pad : {int64_t(0), int64_t(5)}) {
          if (M * (N + pad) > (int64_t(1) << 40)) continue;
          const int64_t stride = N + pad;
          expect_ok(swiglu_fwd(slot(0), slot(1), slot(2), M, N, stride, dtype, nullptr), "swiglu_fwd", M, N);
          expect_ok(swiglu_fwd(slot(0), slot(1), slot(0), M, N, stride, dtype, nullptr), "swiglu_fwd over e", M, N);
          expect_ok(swiglu_bwd(slot(3), slot(0), slot(1), slot(4), slot(5), slot(6), M, N, stride, dtype, nullptr),
                    "swiglu_bwd", M, N);
          expect_ok(swiglu_bwd(slot(3), slot(0), slot(1), slot(3), slot(0), slot(1), M, N, stride, dtype, nullptr),
                    "swiglu_bwd in place", M, N);
        }

  // reductions of tables whose element count would wrap int64: rejected, nothing launched
  const long launches_before = g_launches;
  for (int64_t rows : {int64_t(1) << 61, int64_t(1) << 62, std::numeric_limits<int64_t>::max()})
    for (int64_t N : {int64_t(1), int64_t(4), int64_t(8), int64_t(16384)}) {
      expect(rmsnorm_dgamma_reduce(reinterpret_cast<const float*>(slot(6)), rows, N,
                                   reinterpret_cast<float*>(slot(7)), nullptr) == RMSNORM_E_SHAPE,
             "huge rmsnorm partials table rejected", rows, N);
      expect(layernorm_dwdb_reduce(reinterpret_cast<const float*>(slot(6)), rows, N,
                                   reinterpret_cast<float*>(slot(7)), reinterpret_cast<float*>(slot(10)),
                                   nullptr) == RMSNORM_E_SHAPE,
             "huge layernorm partials tables rejected", rows, N);
    }
  expect(g_launches == launches_before, "no launch for a rejected table");

  expect(rmsn::g_scratch_lookups > 0, "the static scratch was used");
  std::printf("%ld launches checked, %ld checks, %ld bad\n", g_launches, g_checks, g_bad);
  return g_bad ? 1 : 0;
}
