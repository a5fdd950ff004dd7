// Host side of the LayerNorm C ABI declared in include/layernorm.h: argument
// validation, launch planning and the extern "C" entry points.  Validation is
// plain host arithmetic (no HIP call) and finishes before anything is
// launched; on failure every buffer is left untouched.
#include "layernorm.h"

#include <cmath>
#include <cstdint>

#include "host_plan.h"
#include "launch.h"

namespace rmsn {
namespace {

int check_dtype_shape(int64_t M, int64_t N, int64_t stride, int dtype) {
  if (dtype != RMSNORM_F32 && dtype != RMSNORM_BF16 && dtype != RMSNORM_F16) return RMSNORM_E_DTYPE;
  return check_shape(M, N, stride, dtype == RMSNORM_F32 ? RMSNORM_N_MAX : LAYERNORM_N_MAX_16BIT);
}

// Two partial tables (dw, db) of up to partial_rows_bound(M) rows each (rows
// beyond RMSNORM_N_MAX: the wide backward's grid, at most one workgroup per CU).
int64_t ln_workspace_bytes(int64_t M, int64_t N) {
  return 2 * (N > RMSNORM_N_MAX ? wide_partial_rows_bound(M) : partial_rows_bound(M)) * N * 4;
}

int check_ln_bwd(const void* x, const void* weight, const void* dy, const float* mean, const float* rstd,
                 const void* dx, const float* dw, const float* db, const void* workspace, size_t workspace_bytes,
                 int64_t M, int64_t N, int64_t stride, int dtype, bool with_reduce) {
  int st = check_dtype_shape(M, N, stride, dtype);
  if (st) return st;
  if (with_reduce && (!dw || !db)) return RMSNORM_E_NULL;
  if (with_reduce && (!aligned(dw, 4) || !aligned(db, 4))) return RMSNORM_E_ALIGN;
  if (with_reduce && overlap(span(dw, N * 4), span(db, N * 4))) return RMSNORM_E_ALIAS;
  if (M == 0) return RMSNORM_OK;
  if (!x || !weight || !dy || !mean || !rstd || !dx || !workspace) return RMSNORM_E_NULL;
  const int es = elsize(dtype);
  if (!aligned(x, es) || !aligned(weight, es) || !aligned(dy, es) || !aligned(dx, es) || !aligned(mean, 4) ||
      !aligned(rstd, 4) || !aligned(workspace, 4))
    return RMSNORM_E_ALIGN;
  const int64_t need = ln_workspace_bytes(M, N);
  if (workspace_bytes < static_cast<size_t>(need)) return RMSNORM_E_WORKSPACE;
  const int64_t mb = matrix_bytes(M, N, stride, dtype);
  const Span sx = span(x, mb), sdy = span(dy, mb), sdx = span(dx, mb), sg = span(weight, N * es),
             sm = span(mean, M * 4), sr = span(rstd, M * 4), sw = span(workspace, need);
  for (Span o : {sx, sg, sm, sr, sw})
    if (overlap(sdx, o)) return RMSNORM_E_ALIAS;
  if (dx != dy && overlap(sdx, sdy)) return RMSNORM_E_ALIAS;
  for (Span o : {sx, sdy, sg, sm, sr})
    if (overlap(sw, o)) return RMSNORM_E_ALIAS;
  if (with_reduce) {
    for (Span d : {span(dw, N * 4), span(db, N * 4)})
      for (Span o : {sx, sdy, sdx, sg, sm, sr, sw})
        if (overlap(d, o)) return RMSNORM_E_ALIAS;
  }
  return RMSNORM_OK;
}

int launch_ln_bwd_rows_checked(const void* x, const void* weight, const void* dy, const float* mean,
                               const float* rstd, void* dx, void* workspace, int64_t M, int64_t N, int64_t stride,
                               int dtype, int64_t* rows_written, hipStream_t stream) {
  const int vec = choose_vec(dtype, N, stride, {x, weight, dy, dx});
  const bool wide = N > RMSNORM_N_MAX;  // 16-bit rows only (check_dtype_shape)
  const RowPlan p = wide ? plan_ln_wide(true, M, N, vec) : plan_rows(RowOp::kLnBwd, M, N, vec, dtype);
  if (p.iters == 0) return RMSNORM_E_SHAPE;
  LnBwdArgs a{};
  a.x = x;
  a.weight = weight;
  a.dy = dy;
  a.mean = mean;
  a.rstd = rstd;
  a.dx = dx;
  a.partials = static_cast<float*>(workspace);
  a.M = M;
  a.stride = stride;
  a.N = static_cast<int32_t>(N);
  a.nvec = static_cast<int32_t>(N / vec);
  a.inv_n = static_cast<float>(1.0 / static_cast<double>(N));
  a.wpr = p.wpr;
  a.rpb = p.rpb;
  a.row_iters = p.row_iters;
  a.pipeline = wide ? 0 : bwd_pipelined(RowOp::kLnBwd, p, dtype);
  a.partials_nt = !wide && partials_nontemporal(2, p.grid, N);
  a.chunks = wide ? p.iters : 0;
  const int st = hip_status(wide ? launch_ln_bwd_wide(dtype, p, a, stream) : launch_ln_bwd_rows(dtype, p, a, stream));
  if (st == RMSNORM_OK) *rows_written = p.grid;
  return st;
}

int launch_dwdb_reduce_checked(const float* partials, int64_t rows, int64_t N, float* dw, float* db,
                               hipStream_t stream) {
  const bool wide = N % 4 == 0 && aligned(dw, 16) && aligned(db, 16) && (rows == 0 || aligned(partials, 16));
  ReduceArgs a{partials, dw, rows, static_cast<int32_t>(N), db};
  return hip_status(launch_dgamma_reduce(wide ? 4 : 1, 2, a, stream));
}

}  // namespace
}  // namespace rmsn

using namespace rmsn;

extern "C" {

int layernorm_fwd(const void* x, const void* weight, const void* bias, void* y, float* mean, float* rstd, int64_t M,
                  int64_t N, int64_t row_stride, float eps, int dtype, hipStream_t stream) {
  int st = check_dtype_shape(M, N, row_stride, dtype);
  if (st) return st;
  if (!std::isfinite(eps) || !(eps > 0.0f)) return RMSNORM_E_EPS;
  if (M == 0) return RMSNORM_OK;
  if (!x || !weight || !bias || !y || !mean || !rstd) return RMSNORM_E_NULL;
  const int es = elsize(dtype);
  if (!aligned(x, es) || !aligned(weight, es) || !aligned(bias, es) || !aligned(y, es) || !aligned(mean, 4) ||
      !aligned(rstd, 4))
    return RMSNORM_E_ALIGN;
  const int64_t mb = matrix_bytes(M, N, row_stride, dtype);
  const Span sx = span(x, mb), sy = span(y, mb), sw = span(weight, N * es), sb = span(bias, N * es),
             sm = span(mean, M * 4), sr = span(rstd, M * 4);
  for (Span out : {sy, sm, sr})
    for (Span o : {sx, sw, sb})
      if (overlap(out, o)) return RMSNORM_E_ALIAS;
  if (overlap(sy, sm) || overlap(sy, sr) || overlap(sm, sr)) return RMSNORM_E_ALIAS;

  const int vec = choose_vec(dtype, N, row_stride, {x, weight, bias, y});
  const RowPlan p = plan_ln_fwd(M, N, vec, dtype);
  const bool wide = p.wide;
  if (p.iters == 0) return RMSNORM_E_SHAPE;
  LnFwdArgs a{};
  a.x = x;
  a.weight = weight;
  a.bias = bias;
  a.y = y;
  a.mean = mean;
  a.rstd = rstd;
  a.M = M;
  a.stride = row_stride;
  a.N = static_cast<int32_t>(N);
  a.nvec = static_cast<int32_t>(N / vec);
  a.eps = eps;
  a.inv_n = static_cast<float>(1.0 / static_cast<double>(N));
  a.wpr = p.wpr;
  a.rpb = p.rpb;
  a.row_iters = p.row_iters;
  a.chunks = wide ? p.iters : 0;
  return hip_status(wide ? launch_ln_fwd_wide(dtype, p, a, stream) : launch_ln_fwd(dtype, p, a, stream));
}

int layernorm_bwd_workspace_bytes(int64_t M, int64_t N, int dtype, size_t* bytes) {
  if (!bytes) return RMSNORM_E_NULL;
  const int st = check_dtype_shape(M, N, N, dtype);
  if (st) return st;
  *bytes = static_cast<size_t>(ln_workspace_bytes(M, N));
  return RMSNORM_OK;
}

int layernorm_bwd_rows(const void* x, const void* weight, const void* dy, const float* mean, const float* rstd,
                       void* dx, void* workspace, size_t workspace_bytes, int64_t M, int64_t N, int64_t row_stride,
                       int dtype, int64_t* partial_rows, hipStream_t stream) {
  if (!partial_rows) return RMSNORM_E_NULL;
  const int st = check_ln_bwd(x, weight, dy, mean, rstd, dx, nullptr, nullptr, workspace, workspace_bytes, M, N,
                              row_stride, dtype, false);
  if (st) return st;
  *partial_rows = 0;
  if (M == 0) return RMSNORM_OK;
  return launch_ln_bwd_rows_checked(x, weight, dy, mean, rstd, dx, workspace, M, N, row_stride, dtype, partial_rows,
                                    stream);
}

int layernorm_dwdb_reduce(const float* partials, int64_t rows, int64_t N, float* dw, float* db, hipStream_t stream) {
  // two tables of rows x N; bounded by division, as 2 * rows * N could wrap
  if (rows < 0 || N < 1 || N > LAYERNORM_N_MAX_16BIT || rows > RMSNORM_PARTIALS_MAX / (2 * N)) return RMSNORM_E_SHAPE;
  if (!dw || !db || (rows > 0 && !partials)) return RMSNORM_E_NULL;
  if (!aligned(dw, 4) || !aligned(db, 4) || (rows > 0 && !aligned(partials, 4))) return RMSNORM_E_ALIGN;
  const Span sp = span(partials, 2 * rows * N * 4), sw = span(dw, N * 4), sb = span(db, N * 4);
  if (overlap(sw, sb) || (rows > 0 && (overlap(sp, sw) || overlap(sp, sb)))) return RMSNORM_E_ALIAS;
  return launch_dwdb_reduce_checked(partials, rows, N, dw, db, stream);
}

int layernorm_bwd(const void* x, const void* weight, const void* dy, const float* mean, const float* rstd, void* dx,
                  float* dw, float* db, void* workspace, size_t workspace_bytes, int64_t M, int64_t N,
                  int64_t row_stride, int dtype, hipStream_t stream) {
  int st = check_ln_bwd(x, weight, dy, mean, rstd, dx, dw, db, workspace, workspace_bytes, M, N, row_stride, dtype,
                        true);
  if (st) return st;
  int64_t rows = 0;
  if (M > 0) {
    st = launch_ln_bwd_rows_checked(x, weight, dy, mean, rstd, dx, workspace, M, N, row_stride, dtype, &rows, stream);
    if (st) return st;
  }
  return launch_dwdb_reduce_checked(static_cast<const float*>(workspace), rows, N, dw, db, stream);
}

}  // extern "C"
