/*
 * layernorm.h — C ABI of the LayerNorm operations in the MI355X (gfx950)
 * row-normalisation library (librmsnorm.so, beside the RMSNorm entry points
 * of rmsnorm.h, whose dtype codes, status codes and limits it shares).
 *
 * Operations, as defined in the LayerNorm chapter of a Triton tutorial series,
 * "第 07 章:LayerNorm——反向传播与原子锁" (chuoer47.github.io):
 *
 *   forward   mean_i = sum_j x_ij / N
 *             var_i  = sum_j (x_ij - mean_i)^2 / N            (biased; section 1)
 *             rstd_i = 1 / sqrt(var_i + eps)
 *             y_ij   = (x_ij - mean_i) * rstd_i * w_j + b_j
 *   backward  x_hat = (x - mean) * rstd,  g = w * dy             (section 3.0, 3.3)
 *             c1_i = sum_j x_hat_ij g_ij / N,  c2_i = sum_j g_ij / N
 *             dx_ij = (g_ij - (x_hat_ij c1_i + c2_i)) * rstd_i
 *             dw_j = sum_i dy_ij x_hat_ij,  db_j = sum_i dy_ij    (sections 3.3-3.5)
 *
 * The chapter accumulates each row's dw/db contribution into GROUP_SIZE
 * intermediate rows under spin locks, then reduces those rows in a second
 * kernel.  Here the same two stages have no locks: layernorm_bwd_rows writes
 * one fp32 partial row of dw and one of db per workgroup of a persistent
 * grid, layernorm_dwdb_reduce sums them in a fixed order, and layernorm_bwd
 * runs both.
 *
 * Conventions (as in rmsnorm.h): row-major M x N matrices sharing one row
 * stride in elements; dtype (RMSNORM_F32 / RMSNORM_BF16 / RMSNORM_F16)
 * applies to x, weight, bias, y, dy and dx; mean, rstd, dw, db and the
 * partials are fp32.  Arithmetic is fp32 in registers, each 16-bit output
 * rounded to nearest even once.  All pointers are device pointers the
 * caller owns; nothing is allocated and no state is kept; calls are
 * asynchronous on `stream`.  Arguments are validated on the host first; on
 * any error nothing is launched or written and a status is returned.  Results
 * are bitwise deterministic for fixed inputs, shapes and pointer alignments.
 * The status codes are those of rmsnorm.h (RMSNORM_OK, RMSNORM_E_*).
 */
#ifndef LAYERNORM_H
#define LAYERNORM_H

#include "rmsnorm.h"

/* Longest LayerNorm row: the chapter's forward wrapper takes rows of up to
 * 64 KB (Step 2, the wrapper's block-size limit).  bf16 and fp16 rows may have up
 * to 32768 elements (rows beyond 16384 run in chunked kernels, one 1024-thread
 * workgroup per row); fp32 rows, as for RMSNorm, up to RMSNORM_N_MAX = 16384. */
#define LAYERNORM_N_MAX_16BIT 32768

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Forward: y, and the per-row mean and rstd kept for the backward (section 1).
 *
 *   x      [M, N] dtype, read         weight, bias [N] dtype, read
 *   y      [M, N] dtype, written (every element of the M x N view)
 *   mean   [M] fp32, written          rstd [M] fp32, written
 *   row_stride  elements between row starts of x and y (>= N)
 *   eps    finite, > 0; added to the variance under the square root
 * M == 0 is a no-op.  y, mean and rstd must not overlap each other or an input.
 */
int layernorm_fwd(const void* x, const void* weight, const void* bias, void* y, float* mean, float* rstd,
                  int64_t M, int64_t N, int64_t row_stride, float eps, int dtype, hipStream_t stream);

/*
 * Bytes of fp32 workspace layernorm_bwd_rows / layernorm_bwd need for an
 * M x N problem (room for two partial tables of up to min(M, 1024) rows;
 * min(M, 256) rows for N > RMSNORM_N_MAX).  Pure host arithmetic.  *bytes is
 * written only on RMSNORM_OK.
 */
int layernorm_bwd_workspace_bytes(int64_t M, int64_t N, int dtype, size_t* bytes);

/*
 * Backward row pass: dx for every row, and the dw and db contributions
 * (dy * x_hat and dy) summed per workgroup into fp32 partial rows (sections
 * 3.0-3.3).  mean and rstd are read, never recomputed.
 *
 *   x, dy   [M, N] dtype, read          weight [N] dtype, read
 *   mean, rstd  [M] fp32, read (as written by layernorm_fwd with the same x, eps)
 *   dx      [M, N] dtype, written; may be exactly dy (same pointer): each
 *           element of dy is read before it is overwritten
 *   workspace  fp32, at least layernorm_bwd_workspace_bytes(); on return,
 *           with P = *partial_rows, rows [0, P) of N floats hold the dw
 *           partials and rows [P, 2P) the db partials
 *   partial_rows  out: P (0 when M == 0)
 * dx must not overlap x, weight, mean, rstd or the workspace, except dx == dy.
 */
int layernorm_bwd_rows(const void* x, const void* weight, const void* dy, const float* mean, const float* rstd,
                       void* dx, void* workspace, size_t workspace_bytes, int64_t M, int64_t N, int64_t row_stride,
                       int dtype, int64_t* partial_rows, hipStream_t stream);

/*
 * Second stage (sections 3.4-3.5): dw_j = sum_{p < rows} partials[p, j] and
 * db_j = sum_{p < rows} partials[rows + p, j], each in fp32 in a fixed order
 * (sums, not means).
 *
 *   partials  [2 * rows, N] fp32, contiguous, read (may be NULL when rows == 0)
 *   dw, db    [N] fp32, overwritten (zeros when rows == 0)
 * Errors: RMSNORM_E_SHAPE when rows < 0, N outside [1, LAYERNORM_N_MAX_16BIT] or
 * 2 * rows * N > RMSNORM_PARTIALS_MAX; RMSNORM_E_ALIAS when an output overlaps
 * the partials or the other output.
 */
int layernorm_dwdb_reduce(const float* partials, int64_t rows, int64_t N, float* dw, float* db, hipStream_t stream);

/*
 * Full backward: layernorm_bwd_rows followed by layernorm_dwdb_reduce on the
 * same stream.  dw and db [N] fp32 are overwritten (zeros when M == 0).
 * Arguments as above; dw and db must not overlap any other buffer.
 */
int layernorm_bwd(const void* x, const void* weight, const void* dy, const float* mean, const float* rstd, void* dx,
                  float* dw, float* db, void* workspace, size_t workspace_bytes, int64_t M, int64_t N,
                  int64_t row_stride, int dtype, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LAYERNORM_H */
