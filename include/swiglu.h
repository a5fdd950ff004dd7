/*
 * swiglu.h — C ABI of the elementwise SwiGLU forward and backward in the
 * MI355X (gfx950) row-normalisation library (librmsnorm.so; dtype codes,
 * status codes and conventions of rmsnorm.h).
 *
 * Operation, as described in the Unsloth kernel walkthrough "02 · 手写 Triton
 * kernel:RMSNorm / RoPE / SwiGLU", section 5: of the MLP
 * h = silu(X@G) * (X@U), the GEMMs stay with the BLAS library and the
 * elementwise part is fused.
 *   forward   f = e * sigmoid(e) in fp32, cast to dtype, then h = f * g:
 *             h = T(T(f) * g), T = round to nearest even in dtype
 *   backward  from the incoming gradient dh (of h), e and g, one pass writes
 *             h  = T(T(f) * g)                      (recomputed)
 *             df = T(dh * T(f))                     (the gradient of g)
 *             de = T(dh * g * s * (1 + e (1 - s)))  (the gradient of e, s = sigmoid(e))
 *             The page writes them in place over dh, e and g respectively;
 *             here each output may be any one of the inputs (same pointer,
 *             same layout) or separate memory.
 * Arithmetic is fp32 on the stored (rounded) inputs.
 *
 *   e, g, dh, h, df, de  [M, N] of dtype, row-major, sharing one row stride
 *                        (elements, >= N); rows of each are contiguous
 * M == 0 is a no-op.  Errors (nothing is launched): RMSNORM_E_DTYPE,
 * RMSNORM_E_SHAPE (M < 0 or > RMSNORM_M_MAX, N < 1 or > 2^26),
 * RMSNORM_E_STRIDE, RMSNORM_E_NULL, RMSNORM_E_ALIGN, RMSNORM_E_ALIAS (an
 * output shares an element with an input without being that input, or two
 * outputs share an element).  The overlap test is exact for the strided
 * layout, so e and g may be the two interleaved halves of one [M, 2N]
 * buffer (row stride 2N) and an output may be either half.
 */
#ifndef SWIGLU_H
#define SWIGLU_H

#include "rmsnorm.h"

#ifdef __cplusplus
extern "C" {
#endif

int swiglu_fwd(const void* e, const void* g, void* h, int64_t M, int64_t N, int64_t row_stride, int dtype,
               hipStream_t stream);

int swiglu_bwd(const void* dh, const void* e, const void* g, void* h, void* df, void* de, int64_t M, int64_t N,
               int64_t row_stride, int dtype, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SWIGLU_H */
