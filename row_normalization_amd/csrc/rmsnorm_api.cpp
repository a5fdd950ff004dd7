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

#include "host_plan.h"
#include "launch.h"

namespace rmsn {
namespace {

int check_common(int64_t M, int64_t N, int64_t stride, int dtype, int flags) {
  if (dtype != RMSNORM_F32 && dtype != RMSNORM_BF16 && dtype != RMSNORM_F16) return RMSNORM_E_DTYPE;
  if (flags & ~(RMSNORM_GEMMA | RMSNORM_ROUND_NORMED)) return RMSNORM_E_FLAG;
  return check_shape(M, N, stride);
}
// Validation shared by rmsnorm_bwd_rows, rmsnorm_bwd and rmsnorm_bwd_noalloc.
// `dgamma` is null for the row pass alone; `own_scratch` skips the checks of
// the caller's workspace (the no-alloc entry point uses the library's static
// scratch, which no caller buffer can overlap).
int check_bwd(const void* x, const void* gamma, const void* dy, const float* rstd, const void* dx, const float* dgamma,
              const void* workspace, size_t workspace_bytes, int64_t M, int64_t N, int64_t stride, int dtype, int flags,
              bool with_dgamma, int64_t* rows_written, bool own_scratch = false) {
  int st = check_common(M, N, stride, dtype, flags);
  if (st) return st;
  if (with_dgamma && !dgamma) return RMSNORM_E_NULL;
  if (with_dgamma && !aligned(dgamma, 4)) return RMSNORM_E_ALIGN;
  *rows_written = 0;
  if (M == 0) return RMSNORM_OK;
  if (!x || !gamma || !dy || !rstd || !dx || (!workspace && !own_scratch)) return RMSNORM_E_NULL;
  const int es = elsize(dtype);
  if (!aligned(x, es) || !aligned(gamma, es) || !aligned(dy, es) || !aligned(dx, es) || !aligned(rstd, 4) ||
      !aligned(workspace, 4))
    return RMSNORM_E_ALIGN;
  const int64_t need = own_scratch ? 0 : partial_rows_bound(M) * N * 4;
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

RowPlan bwd_plan(const void* x, const void* gamma, const void* dy, const void* dx, int64_t M, int64_t N,
                 int64_t stride, int dtype) {
  const int vec = choose_vec(dtype, N, stride, {x, gamma, dy, dx});
  return plan_rows(RowOp::kRmsBwd, M, N, vec, dtype);
}

int launch_bwd_rows_checked(const void* x, const void* gamma, const void* dy, const float* rstd, void* dx,
                            void* workspace, int64_t M, int64_t N, int64_t stride, int dtype, int flags,
                            int64_t* rows_written, hipStream_t stream) {
  const RowPlan p = bwd_plan(x, gamma, dy, dx, M, N, stride, dtype);
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
  a.nvec = static_cast<int32_t>(N / p.vec);
  a.inv_n = static_cast<float>(1.0 / static_cast<double>(N));
  a.w_off = (flags & RMSNORM_GEMMA) ? 1.0f : 0.0f;
  a.wpr = p.wpr;
  a.rpb = p.rpb;
  a.row_iters = p.row_iters;
  a.pipeline = bwd_pipelined(RowOp::kRmsBwd, p, dtype);
  a.partials_nt = partials_nontemporal(1, p.grid, N);
  const int st = hip_status(launch_bwd_rows(dtype, p, a, stream));
  if (st == RMSNORM_OK) *rows_written = p.grid;
  return st;
}

int launch_reduce_checked(const float* partials, int64_t rows, int64_t N, float* dgamma, hipStream_t stream) {
  const int vec = (N % 4 == 0 && aligned(dgamma, 16) && (rows == 0 || aligned(partials, 16))) ? 4 : 1;
  ReduceArgs a{partials, dgamma, rows, static_cast<int32_t>(N), nullptr};
  return hip_status(launch_dgamma_reduce(vec, 1, a, stream));
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
  const RowPlan p = plan_rows(RowOp::kRmsFwd, M, N, vec, dtype);
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
  a.first_row_early = fwd_first_row_early(p);
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
  // the table bound is tested by division: rows * N could wrap for huge rows
  if (rows < 0 || N < 1 || N > RMSNORM_N_MAX || rows > RMSNORM_PARTIALS_MAX / N) return RMSNORM_E_SHAPE;
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

int rmsnorm_bwd_noalloc(const void* x, const void* gamma, const void* dy, const float* rstd, void* dx, float* dgamma,
                        int64_t M, int64_t N, int64_t row_stride, int dtype, int flags, hipStream_t stream) {
  int64_t rows = 0;
  int st = check_bwd(x, gamma, dy, rstd, dx, dgamma, nullptr, 0, M, N, row_stride, dtype, flags, true, &rows, true);
  if (st) return st;
  void* scratch = nullptr;
  if (M > 0) {
    const RowPlan p = bwd_plan(x, gamma, dy, dx, M, N, row_stride, dtype);
    if (p.iters == 0) return RMSNORM_E_SHAPE;
    if (p.grid > RMSNORM_STATIC_SCRATCH_BYTES / (N * 4)) return RMSNORM_E_SCRATCH;
    st = hip_status(static_scratch(&scratch));
    if (st) return st;
    st = launch_bwd_rows_checked(x, gamma, dy, rstd, dx, scratch, M, N, row_stride, dtype, flags, &rows, stream);
    if (st) return st;
  }
  return launch_reduce_checked(static_cast<const float*>(scratch), rows, N, dgamma, stream);
}

const char* rmsnorm_status_string(int status) {
  switch (status) {
    case RMSNORM_OK: return "ok";
    case RMSNORM_E_NULL: return "a required pointer is NULL";
    case RMSNORM_E_SHAPE: return "invalid shape (outside the entry point's documented limits, e.g. 1 <= N <= RMSNORM_N_MAX)";
    case RMSNORM_E_STRIDE: return "row stride smaller than N";
    case RMSNORM_E_ALIGN: return "a pointer is not aligned to its element size";
    case RMSNORM_E_DTYPE: return "unsupported dtype (need RMSNORM_F32, RMSNORM_BF16 or RMSNORM_F16)";
    case RMSNORM_E_EPS: return "eps must be finite and > 0";
    case RMSNORM_E_ALIAS: return "an output overlaps another buffer (beyond the exact in-place cases the entry point allows)";
    case RMSNORM_E_WORKSPACE: return "workspace smaller than the matching *_bwd_workspace_bytes() size";
    case RMSNORM_E_FLAG: return "flags may only combine RMSNORM_GEMMA and RMSNORM_ROUND_NORMED";
    case RMSNORM_E_HIP: return "HIP kernel launch failed";
    case RMSNORM_E_SCRATCH:
      return "the launch plan needs more partial rows than the static scratch holds (RMSNORM_STATIC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"
