// Host side of the C ABI declared in include/rmsnorm.h: argument validation,
// launch planning and the extern "C" entry points.  Validation is plain host
// arithmetic on the arguments (no HIP call), finishes before anything is
// launched, and on failure leaves every buffer untouched.
#include "rmsnorm.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <initializer_list>
#include <limits>

#include "launch.h"

namespace rmsn {
namespace {

// Launch shape.  A row group spans as many waves as it takes for each lane
// to hold kLaneVectors 16-byte vectors of every row operand; workgroups hold
// about kBlockWaves waves (several row groups when rows are short).  Measured
// on MI355X at M=16384, N=8192 bf16: two vectors per lane and eight waves per
// row beat both fewer, fatter lanes and whole-row-per-wave layouts, for the
// forward and the backward alike.
constexpr int kLaneVectors = 2;
constexpr int kBlockWaves = 8;
constexpr int kFwdRowWaves = 8;
// The backward grid is persistent: a whole number of workgroups on each of
// the 256 compute units (a power of two, so that every CU gets the same
// count), about kBwdResidentWaves waves per CU, every workgroup taking a fixed
// share of the rows.  Each workgroup writes one fp32 partial row of dgamma.
// (A grid that does not divide evenly over the CUs leaves a tail: 819
// workgroups for N = 5120 ran 20 % slower than 512.)
constexpr int64_t kComputeUnits = 256;
constexpr int64_t kBwdResidentWaves = 16;
// Upper bound on the backward grid, hence on the partial rows a workspace
// must hold (rmsnorm_bwd_workspace_bytes promises this many rows at most).
constexpr int64_t kBwdGridMax = 1024;
// The forward grid is not persistent; it is only capped so that the grid
// dimension stays small (rows beyond it are taken in further steps).
constexpr int64_t kFwdGridMax = 1 << 20;
// Register budget per lane for the row data, in 32-bit registers (of the 128
// a lane of a 1024-thread workgroup may use): the forward holds x and gamma
// packed; the backward holds x and dy packed plus, per column it owns, the
// fp32 weight and dgamma partial.
constexpr int kLaneDataRegs = 96;

int elsize(int dtype) { return dtype == RMSNORM_F32 ? 4 : 2; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned(const void* p, int64_t bytes) { return reinterpret_cast<uintptr_t>(p) % static_cast<uintptr_t>(bytes) == 0; }

// [p, p + len) for a byte range; empty ranges never overlap.
struct Span {
  uintptr_t lo;
  uintptr_t len;
};
Span span(const void* p, int64_t bytes) { return {reinterpret_cast<uintptr_t>(p), static_cast<uintptr_t>(bytes)}; }
bool overlap(Span a, Span b) { return a.len && b.len && a.lo < b.lo + b.len && b.lo < a.lo + a.len; }

int64_t matrix_bytes(int64_t M, int64_t N, int64_t stride, int dtype) {
  return M == 0 ? 0 : ((M - 1) * stride + N) * elsize(dtype);
}

int check_common(int64_t M, int64_t N, int64_t stride, int dtype, int flags) {
  if (dtype != RMSNORM_F32 && dtype != RMSNORM_BF16 && dtype != RMSNORM_F16) return RMSNORM_E_DTYPE;
  if (flags & ~(RMSNORM_GEMMA | RMSNORM_ROUND_NORMED)) return RMSNORM_E_FLAG;
  if (M < 0 || M > RMSNORM_M_MAX || N < 1 || N > RMSNORM_N_MAX) return RMSNORM_E_SHAPE;
  if (stride < N) return RMSNORM_E_STRIDE;
  // element offsets must stay well inside int64 even for the last row
  if (M > 0 && stride > (std::numeric_limits<int64_t>::max() / 8) / M) return RMSNORM_E_SHAPE;
  return RMSNORM_OK;
}

// Widest vector (up to 16 bytes) that every pointer, N and the stride allow.
int choose_vec(int dtype, int64_t N, int64_t stride, std::initializer_list<const void*> ptrs) {
  const int es = elsize(dtype);
  for (int vec = 16 / es; vec > 1; vec /= 2) {
    bool ok = N % vec == 0 && stride % vec == 0;
    for (const void* p : ptrs) ok = ok && aligned(p, int64_t(vec) * es);
    if (ok) return vec;
  }
  return 1;
}

// Waves per row and vectors per lane: among 1..16 waves per row and the
// compiled register-array lengths, the shape that wastes the fewest lanes;
// ties go to the length nearest `target` vectors per lane, then to fewer waves.
bool row_shape(int64_t nvec, int iters_cap, int target, int* wpr, int* iters) {
  int64_t best_waste = -1;
  int best_dist = 0;
  for (int w = 1; w <= kMaxBlockWaves; ++w) {
    for (int it : kItersSet) {
      if (it > iters_cap || int64_t(it) * kWave * w < nvec) continue;
      const int64_t waste = int64_t(it) * kWave * w - nvec;
      const int dist = it > target ? it - target : target - it;
      if (best_waste < 0 || waste < best_waste || (waste == best_waste && dist < best_dist)) {
        best_waste = waste;
        best_dist = dist;
        *wpr = w;
        *iters = it;
      }
    }
  }
  return best_waste >= 0;
}

// Elements per lane the register budget allows.
int lane_elems_cap(int dtype, bool backward) {
  const int es = elsize(dtype);
  // registers per element, in quarters: packed operands (es each), fp32 values (4 each)
  return backward ? kLaneDataRegs * 4 / (2 * es + 8) : kLaneDataRegs * 4 / (2 * es);
}

RowPlan plan_rows(int64_t M, int64_t N, int vec, int dtype, bool backward) {
  RowPlan p{};
  p.vec = vec;
  const int64_t nvec = N / vec;
  const int cap = std::min(kItersMax, std::max(1, lane_elems_cap(dtype, backward) / vec));
  // The forward prefers rows of at most kFwdRowWaves waves, with more vectors
  // per lane beyond that (measured at N = 16384 bf16: 8 waves x 4 vectors ran
  // 4 % faster than 16 x 2); the backward keeps kLaneVectors.
  const int target =
      backward ? kLaneVectors : static_cast<int>(std::max<int64_t>(kLaneVectors, ceil_div(nvec, int64_t(kWave) * kFwdRowWaves)));
  if (!row_shape(nvec, cap, target, &p.wpr, &p.iters)) {
    p.iters = 0;  // cannot happen for N <= RMSNORM_N_MAX
    return p;
  }
  p.rpb = std::max(1, kBlockWaves / p.wpr);
  const int64_t groups = ceil_div(M, p.rpb);
  int64_t per_cu = 1;
  while (per_cu * 2 * p.wpr * p.rpb <= kBwdResidentWaves) per_cu *= 2;
  const int64_t grid_cap = backward ? std::min(kBwdGridMax, kComputeUnits * per_cu) : kFwdGridMax;
  p.grid = std::max<int64_t>(1, std::min(groups, grid_cap));
  p.row_iters = ceil_div(groups, p.grid);
  return p;
}

int64_t partial_rows_bound(int64_t M) { return std::min(M, kBwdGridMax); }

int hip_status(hipError_t e) { return e == hipSuccess ? RMSNORM_OK : RMSNORM_E_HIP; }

// Validation shared by rmsnorm_bwd_rows and rmsnorm_bwd.  `dgamma` is null
// for the row pass alone.
int check_bwd(const void* x, const void* gamma, const void* dy, const float* rstd, const void* dx, const float* dgamma,
              const void* workspace, size_t workspace_bytes, int64_t M, int64_t N, int64_t stride, int dtype, int flags,
              bool with_dgamma, int64_t* rows_written) {
  int st = check_common(M, N, stride, dtype, flags);
  if (st) return st;
  if (with_dgamma && !dgamma) return RMSNORM_E_NULL;
  if (with_dgamma && !aligned(dgamma, 4)) return RMSNORM_E_ALIGN;
  *rows_written = 0;
  if (M == 0) return RMSNORM_OK;
  if (!x || !gamma || !dy || !rstd || !dx || !workspace) return RMSNORM_E_NULL;
  const int es = elsize(dtype);
  if (!aligned(x, es) || !aligned(gamma, es) || !aligned(dy, es) || !aligned(dx, es) || !aligned(rstd, 4) ||
      !aligned(workspace, 4))
    return RMSNORM_E_ALIGN;
  const int64_t need = partial_rows_bound(M) * N * 4;
  if (workspace_bytes < static_cast<size_t>(need)) return RMSNORM_E_WORKSPACE;
  const int64_t mb = matrix_bytes(M, N, stride, dtype);
  const Span sx = span(x, mb), sdy = span(dy, mb), sdx = span(dx, mb), sg = span(gamma, N * es),
             sr = span(rstd, M * 4), sw = span(workspace, need);
  if (overlap(sdx, sx) || overlap(sdx, sg) || overlap(sdx, sr) || overlap(sdx, sw)) return RMSNORM_E_ALIAS;
  if (dx != dy && overlap(sdx, sdy)) return RMSNORM_E_ALIAS;
  if (overlap(sw, sx) || overlap(sw, sdy) || overlap(sw, sg) || overlap(sw, sr)) return RMSNORM_E_ALIAS;
  if (with_dgamma) {
    const Span sd = span(dgamma, N * 4);
    if (overlap(sd, sx) || overlap(sd, sdy) || overlap(sd, sdx) || overlap(sd, sg) || overlap(sd, sr) ||
        overlap(sd, sw))
      return RMSNORM_E_ALIAS;
  }
  return RMSNORM_OK;
}

int launch_bwd_rows_checked(const void* x, const void* gamma, const void* dy, const float* rstd, void* dx,
                            void* workspace, int64_t M, int64_t N, int64_t stride, int dtype, int flags,
                            int64_t* rows_written, hipStream_t stream) {
  const int vec = choose_vec(dtype, N, stride, {x, gamma, dy, dx});
  const RowPlan p = plan_rows(M, N, vec, dtype, true);
  if (p.iters == 0) return RMSNORM_E_SHAPE;
  BwdArgs a{};
  a.x = x;
  a.gamma = gamma;
  a.dy = dy;
  a.rstd = rstd;
  a.dx = dx;
  a.partials = static_cast<float*>(workspace);
  a.M = M;
  a.stride = stride;
  a.N = static_cast<int32_t>(N);
  a.nvec = static_cast<int32_t>(N / vec);
  a.inv_n = static_cast<float>(1.0 / static_cast<double>(N));
  a.w_off = (flags & RMSNORM_GEMMA) ? 1.0f : 0.0f;
  a.wpr = p.wpr;
  a.rpb = p.rpb;
  a.row_iters = p.row_iters;
  const int st = hip_status(launch_bwd_rows(dtype, p, a, stream));
  if (st == RMSNORM_OK) *rows_written = p.grid;
  return st;
}

int launch_reduce_checked(const float* partials, int64_t rows, int64_t N, float* dgamma, hipStream_t stream) {
  const int vec = (N % 4 == 0 && aligned(dgamma, 16) && (rows == 0 || aligned(partials, 16))) ? 4 : 1;
  ReduceArgs a{partials, dgamma, rows, static_cast<int32_t>(N)};
  return hip_status(launch_dgamma_reduce(vec, a, stream));
}

}  // namespace
}  // namespace rmsn

using namespace rmsn;

extern "C" {

int rmsnorm_fwd(const void* x, const void* gamma, void* y, float* rstd, int64_t M, int64_t N, int64_t row_stride,
                float eps, int dtype, int flags, hipStream_t stream) {
  int st = check_common(M, N, row_stride, dtype, flags);
  if (st) return st;
  if (!std::isfinite(eps) || !(eps > 0.0f)) return RMSNORM_E_EPS;
  if (M == 0) return RMSNORM_OK;
  if (!x || !gamma || !y || !rstd) return RMSNORM_E_NULL;
  const int es = elsize(dtype);
  if (!aligned(x, es) || !aligned(gamma, es) || !aligned(y, es) || !aligned(rstd, 4)) return RMSNORM_E_ALIGN;
  const int64_t mb = matrix_bytes(M, N, row_stride, dtype);
  const Span sx = span(x, mb), sy = span(y, mb), sg = span(gamma, N * es), sr = span(rstd, M * 4);
  if (overlap(sy, sx) || overlap(sy, sg) || overlap(sy, sr) || overlap(sr, sx) || overlap(sr, sg))
    return RMSNORM_E_ALIAS;

  const int vec = choose_vec(dtype, N, row_stride, {x, gamma, y});
  const RowPlan p = plan_rows(M, N, vec, dtype, false);
  if (p.iters == 0) return RMSNORM_E_SHAPE;
  FwdArgs a{};
  a.x = x;
  a.gamma = gamma;
  a.y = y;
  a.rstd = rstd;
  a.M = M;
  a.stride = row_stride;
  a.N = static_cast<int32_t>(N);
  a.nvec = static_cast<int32_t>(N / vec);
  a.eps = eps;
  a.inv_n = static_cast<float>(1.0 / static_cast<double>(N));
  a.w_off = (flags & RMSNORM_GEMMA) ? 1.0f : 0.0f;
  a.wpr = p.wpr;
  a.rpb = p.rpb;
  a.row_iters = p.row_iters;
  a.round_normed = (flags & RMSNORM_ROUND_NORMED) && dtype != RMSNORM_F32;
  return hip_status(launch_fwd(dtype, p, a, stream));
}

int rmsnorm_bwd_workspace_bytes(int64_t M, int64_t N, int dtype, size_t* bytes) {
  if (!bytes) return RMSNORM_E_NULL;
  const int st = check_common(M, N, N, dtype, 0);
  if (st) return st;
  *bytes = static_cast<size_t>(partial_rows_bound(M) * N * 4);
  return RMSNORM_OK;
}

int rmsnorm_bwd_rows(const void* x, const void* gamma, const void* dy, const float* rstd, void* dx, void* workspace,
                     size_t workspace_bytes, int64_t M, int64_t N, int64_t row_stride, int dtype, int flags,
                     int64_t* partial_rows, hipStream_t stream) {
  if (!partial_rows) return RMSNORM_E_NULL;
  int64_t rows = 0;
  const int st = check_bwd(x, gamma, dy, rstd, dx, nullptr, workspace, workspace_bytes, M, N, row_stride, dtype, flags,
                           false, &rows);
  if (st) return st;
  *partial_rows = 0;
  if (M == 0) return RMSNORM_OK;
  return launch_bwd_rows_checked(x, gamma, dy, rstd, dx, workspace, M, N, row_stride, dtype, flags, partial_rows,
                                 stream);
}

int rmsnorm_dgamma_reduce(const float* partials, int64_t rows, int64_t N, float* dgamma, hipStream_t stream) {
  if (rows < 0 || N < 1 || N > RMSNORM_N_MAX || rows * N > RMSNORM_PARTIALS_MAX) return RMSNORM_E_SHAPE;
  if (!dgamma || (rows > 0 && !partials)) return RMSNORM_E_NULL;
  if (!aligned(dgamma, 4) || (rows > 0 && !aligned(partials, 4))) return RMSNORM_E_ALIGN;
  if (rows > 0 && overlap(span(partials, rows * N * 4), span(dgamma, N * 4))) return RMSNORM_E_ALIAS;
  return launch_reduce_checked(partials, rows, N, dgamma, stream);
}

int rmsnorm_bwd(const void* x, const void* gamma, const void* dy, const float* rstd, void* dx, float* dgamma,
                void* workspace, size_t workspace_bytes, int64_t M, int64_t N, int64_t row_stride, int dtype,
                int flags, hipStream_t stream) {
  int64_t rows = 0;
  int st = check_bwd(x, gamma, dy, rstd, dx, dgamma, workspace, workspace_bytes, M, N, row_stride, dtype, flags, true,
                     &rows);
  if (st) return st;
  if (M > 0) {
    st = launch_bwd_rows_checked(x, gamma, dy, rstd, dx, workspace, M, N, row_stride, dtype, flags, &rows, stream);
    if (st) return st;
  }
  return launch_reduce_checked(static_cast<const float*>(workspace), rows, N, dgamma, stream);
}

const char* rmsnorm_status_string(int status) {
  switch (status) {
    case RMSNORM_OK: return "ok";
    case RMSNORM_E_NULL: return "a required pointer is NULL";
    case RMSNORM_E_SHAPE: return "invalid shape (need M >= 0 and 1 <= N <= RMSNORM_N_MAX)";
    case RMSNORM_E_STRIDE: return "row stride smaller than N";
    case RMSNORM_E_ALIGN: return "a pointer is not aligned to its element size";
    case RMSNORM_E_DTYPE: return "unsupported dtype (need RMSNORM_F32, RMSNORM_BF16 or RMSNORM_F16)";
    case RMSNORM_E_EPS: return "eps must be finite and > 0";
    case RMSNORM_E_ALIAS: return "an output overlaps another buffer (only dx == dy is allowed)";
    case RMSNORM_E_WORKSPACE: return "workspace smaller than rmsnorm_bwd_workspace_bytes()";
    case RMSNORM_E_FLAG: return "flags may only combine RMSNORM_GEMMA and RMSNORM_ROUND_NORMED";
    case RMSNORM_E_HIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
