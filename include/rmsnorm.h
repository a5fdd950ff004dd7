/*
 * rmsnorm.h — C ABI of the MI355X (gfx950) fused RMSNorm library.
 *
 * Operations, as defined on the Triton RMSNorm tutorial "Hướng dẫn Triton
 * RMSNorm: kernel, backward và…" (partitech.com) and the Unsloth kernel
 * walkthrough "02 · 手写 Triton kernel:RMSNorm / RoPE / SwiGLU" (section 3):
 *
 *   forward   r_i  = 1 / sqrt(mean_j x_ij^2 + eps)          (eps under the root)
 *             y_ij = x_ij * r_i * w_j                       (w = gamma, or 1 + gamma
 *                                                            for the Gemma variant)
 *   backward  u_ij = dy_ij * w_j,  m_i = mean_j u_ij x_ij
 *             dx_ij = r_i u_ij - x_ij r_i^3 m_i
 *             dgamma_j = sum_i dy_ij x_ij r_i               (a sum over rows, not a mean)
 *
 * The tutorial splits the backward into a row pass ("backward_rows": dx plus
 * per-row dgamma contributions) and a column reduction
 * ("reduce_gamma_gradient"); this library keeps that split as
 * rmsnorm_bwd_rows + rmsnorm_dgamma_reduce, with the contributions summed per
 * workgroup first (one fp32 partial row per workgroup instead of one per
 * matrix row), and rmsnorm_bwd runs both.
 *
 * Conventions for every entry point:
 *  - Matrices are row-major M x N with a row stride (in elements) shared by
 *    all matrices of one call; elements of a row are contiguous.
 *  - dtype is RMSNORM_F32, RMSNORM_BF16 or RMSNORM_F16 and applies to x,
 *    gamma, y, dy and dx.  rstd (the saved r) is always fp32[M]; dgamma and
 *    the partials are always fp32.  Arithmetic is fp32 in registers; each
 *    bf16/fp16 output is rounded to nearest even, once (twice for y with
 *    RMSNORM_ROUND_NORMED).
 *  - All pointers are device pointers to memory the caller owns (for example
 *    PyTorch tensors).  The library allocates nothing and keeps no state
 *    between calls (the one exception is rmsnorm_bwd_noalloc's static
 *    scratch, below); calls are asynchronous on `stream` (0 = the null
 *    stream) and their outputs are valid once the stream has reached them.
 *  - Arguments are validated on the host before anything is launched.  On any
 *    error nothing is launched and nothing is written.  Status codes are
 *    returned, never thrown.  There is no fallback path of any kind.
 *  - 16-byte vector loads are used when every base pointer, N and the row
 *    stride allow them; otherwise narrower loads (down to one element) — the
 *    results are the same either way up to fp32 summation order.
 *  - Results are deterministic: the same inputs, shapes and pointer
 *    alignments give bitwise identical outputs on every run (fixed row-to-
 *    workgroup assignment, fixed summation order, no atomics on data).
 */
#ifndef RMSNORM_H
#define RMSNORM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { RMSNORM_F32 = 0, RMSNORM_BF16 = 1, RMSNORM_F16 = 2 } rmsnorm_dtype;

/* Bits of the `flags` argument.
 *  RMSNORM_GEMMA         the weight is applied as (1 + gamma), formed in fp32
 *                        (Unsloth walkthrough, section 3: the Gemma variant).
 *  RMSNORM_ROUND_NORMED  forward only: round x*r to the I/O dtype before the
 *                        weight multiply, y = T(T(x*r) * w), the order of the
 *                        Hugging Face RMSNorm the walkthrough follows
 *                        ("normed.to(W.dtype)" before "* W"); without it y is
 *                        rounded once, y = T(x*r*w).  No effect for fp32.
 *                        The backward accepts and ignores it (its formula
 *                        treats the rounding as the identity). */
enum { RMSNORM_GEMMA = 1, RMSNORM_ROUND_NORMED = 2 };

typedef enum {
  RMSNORM_OK = 0,
  RMSNORM_E_NULL = -1,      /* a required pointer is NULL (only checked when M > 0, or N for dgamma) */
  RMSNORM_E_SHAPE = -2,     /* M outside [0, RMSNORM_M_MAX], N outside [1, RMSNORM_N_MAX], or a bad
                               partials table (rows < 0 or rows * N > RMSNORM_PARTIALS_MAX) */
  RMSNORM_E_STRIDE = -3,    /* row_stride < N */
  RMSNORM_E_ALIGN = -4,     /* a pointer is not aligned to its element size */
  RMSNORM_E_DTYPE = -5,     /* dtype is not RMSNORM_F32 / RMSNORM_BF16 / RMSNORM_F16 */
  RMSNORM_E_EPS = -6,       /* eps is not finite or not > 0 */
  RMSNORM_E_ALIAS = -7,     /* an output overlaps another buffer (for these entry points dx == dy is the
                               one allowed case; layernorm.h, rope.h and swiglu.h state theirs) */
  RMSNORM_E_WORKSPACE = -8, /* workspace smaller than rmsnorm_bwd_workspace_bytes() (or
                               layernorm_bwd_workspace_bytes() for the LayerNorm backward) */
  RMSNORM_E_FLAG = -9,      /* flags has a bit other than RMSNORM_GEMMA | RMSNORM_ROUND_NORMED */
  RMSNORM_E_HIP = -10,      /* a HIP launch failed */
  RMSNORM_E_SCRATCH = -11   /* rmsnorm_bwd_noalloc: the problem needs more partial rows than the
                               library's static scratch holds (RMSNORM_STATIC_SCRATCH_BYTES) */
} rmsnorm_status;

/* Largest supported row length (columns), row count, and partials table
 * (rows * N floats) accepted by rmsnorm_dgamma_reduce.  The kernels address
 * a row, the saved r and the partials through 32-bit byte offsets. */
#define RMSNORM_N_MAX 16384
#define RMSNORM_M_MAX (1LL << 29)
#define RMSNORM_PARTIALS_MAX (1LL << 29)

/* Size of the static device scratch behind rmsnorm_bwd_noalloc (one copy per
 * GPU the library runs on, held until the process ends).  Every launch plan
 * of the backward row pass needs at most 17.5 MiB of partial rows (fp32
 * N = 8960 at 512 partial rows), so every accepted shape fits. */
#define RMSNORM_STATIC_SCRATCH_BYTES (32LL << 20)

/*
 * Forward: y = x * r * w and the saved r (tutorial, "Vấn đề và công thức tham
 * chiếu" and "Forward Triton: một hàng, một chương trình"; Gemma weight from
 * the Unsloth walkthrough, section 3).
 *
 *   x      [M, N] dtype, read         gamma [N] dtype, read
 *   y      [M, N] dtype, written (every element of the M x N view; the padding
 *          between rows of a strided view is not touched)
 *   rstd   [M] fp32, written: r_i, for rmsnorm_bwd_rows
 *   row_stride  elements between row starts of x and y (>= N)
 *   eps    finite, > 0; added to the mean of squares under the square root
 *   flags  RMSNORM_GEMMA: w = 1 + gamma (formed in fp32), else w = gamma;
 *          RMSNORM_ROUND_NORMED: the rounding order described above
 * M == 0 is a no-op.  y must not overlap x, gamma or rstd.
 */
int rmsnorm_fwd(const void* x, const void* gamma, void* y, float* rstd, int64_t M, int64_t N,
                int64_t row_stride, float eps, int dtype, int flags, hipStream_t stream);

/*
 * Size in bytes of the fp32 partials workspace rmsnorm_bwd_rows / rmsnorm_bwd
 * need for an M x N problem of this dtype (an upper bound on the partial rows
 * actually written, times N * 4).  Pure host arithmetic, no HIP call.
 * Returns a status; *bytes is written only on RMSNORM_OK.
 */
int rmsnorm_bwd_workspace_bytes(int64_t M, int64_t N, int dtype, size_t* bytes);

/*
 * Backward row pass: dx for every row and the dgamma contributions dy*x*r
 * summed per workgroup into fp32 partial rows (tutorial, "Backward đầu vào:
 * giữ đúng N", "Lập phương của r từ đâu?" and "Reduce dgamma không có race
 * khi ghi").  r is taken from rstd, never recomputed.
 *
 *   x, dy  [M, N] dtype, read          gamma [N] dtype, read
 *   rstd   [M] fp32, read (as written by rmsnorm_fwd with the same x, eps)
 *   dx     [M, N] dtype, written; may be exactly dy (same pointer) for an
 *          in-place backward — each element of dy is read before it is
 *          overwritten, and nothing later reads dy
 *   workspace  fp32, at least rmsnorm_bwd_workspace_bytes(); on return its
 *          first (*partial_rows) rows of N floats hold the partial sums
 *   partial_rows  out: number of partial rows written (0 when M == 0)
 *   flags  as in rmsnorm_fwd (RMSNORM_GEMMA selects w = 1 + gamma)
 * dx must not overlap x, gamma, rstd or the workspace, except dx == dy.
 */
int rmsnorm_bwd_rows(const void* x, const void* gamma, const void* dy, const float* rstd, void* dx,
                     void* workspace, size_t workspace_bytes, int64_t M, int64_t N, int64_t row_stride,
                     int dtype, int flags, int64_t* partial_rows, hipStream_t stream);

/*
 * Second stage of the weight gradient: dgamma_j = sum over the `rows` partial
 * rows of partials[p, j], summed in fp32 in a fixed order (tutorial, "Reduce
 * dgamma không có race khi ghi" and "Tổng không phải trung bình": a sum, no
 * division by the row count).
 *
 *   partials  [rows, N] fp32, row-major and contiguous, read (may be NULL when rows == 0)
 *   dgamma    [N] fp32, overwritten (rows == 0 gives zeros)
 */
int rmsnorm_dgamma_reduce(const float* partials, int64_t rows, int64_t N, float* dgamma, hipStream_t stream);

/*
 * Full backward: rmsnorm_bwd_rows followed by rmsnorm_dgamma_reduce on the
 * same stream.  dgamma [N] fp32 is overwritten (zeros when M == 0), never
 * accumulated into; it must not overlap any other buffer.
 */
int rmsnorm_bwd(const void* x, const void* gamma, const void* dy, const float* rstd, void* dx, float* dgamma,
                void* workspace, size_t workspace_bytes, int64_t M, int64_t N, int64_t row_stride, int dtype,
                int flags, hipStream_t stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * full backward as rmsnorm_bwd (same kernels, same launch plan, bitwise the
 * same dx and dgamma), with the partial rows kept in a static device array
 * of the library, RMSNORM_STATIC_SCRATCH_BYTES per GPU, instead of a
 * caller's workspace.  Calls no hipMalloc, hipFree or allocating routine; the
 * first call on a device resolves that device's copy of the array (a symbol
 * lookup), later calls reuse it.
 *
 * The array is shared by every call on a GPU and holds the last call's
 * partial rows; the row pass overwrites every row it uses, so nothing needs
 * clearing.  Calls that overlap on one GPU (concurrent streams, or other
 * threads) race on it: serialise them.  Arguments and errors as rmsnorm_bwd,
 * without the workspace; RMSNORM_E_SCRATCH if the launch plan's partial rows
 * (rows x N x 4 bytes) exceed RMSNORM_STATIC_SCRATCH_BYTES (no shape the
 * current planner emits does), RMSNORM_E_HIP if the symbol lookup fails.
 */
int rmsnorm_bwd_noalloc(const void* x, const void* gamma, const void* dy, const float* rstd, void* dx,
                        float* dgamma, int64_t M, int64_t N, int64_t row_stride, int dtype, int flags,
                        hipStream_t stream);

/* A static, human-readable description of a status code. */
const char* rmsnorm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* RMSNORM_H */
