/*
 * rope.h — C ABI of the rotary position embedding (RoPE) in the MI355X
 * (gfx950) row-normalisation library (librmsnorm.so; dtype codes, status
 * codes and conventions of rmsnorm.h).
 *
 * Operation, as described in the Unsloth kernel walkthrough "02 · 手写 Triton
 * kernel:RMSNorm / RoPE / SwiGLU", section 4: every pair of dimensions of a
 * head is rotated by its token's position angle,
 *     q1' = q1 cos - q2 sin,   q2' = q2 cos + q1 sin,
 * in place.  The rotation is invertible, so the backward is the same kernel
 * with sin negated, applied in place to the incoming gradient; nothing is
 * saved between the two.  As on the page, one work item handles a group of
 * four heads of one token, so each cos/sin value is loaded once for the four.
 *
 * The pairs are the two halves of a head: q1 = q[..., :D/2], q2 = q[..., D/2:]
 * (the half-split pairing of the Hugging Face Llama code the walkthrough
 * patches).  Arithmetic is fp32; each output is rounded once (to nearest even).
 *
 *   q          [tokens, heads, head_dim] of dtype, read and written in place;
 *              the heads of a token are contiguous (head stride head_dim),
 *              tokens are token_stride elements apart (>= heads * head_dim)
 *   head_dim   even, 2 .. 1024
 *   cos, sin   [table_rows, head_dim / 2] fp32, contiguous, read
 *   positions  int32 [tokens] (the table row of each token), or NULL: token t
 *              then uses row t mod seq_len (seq_len >= 1 and <= table_rows).
 *              A position outside [0, table_rows) reads cos = sin = 0 (the
 *              loads are range-checked by the hardware) and so writes zeros.
 * tokens == 0 is a no-op.  Errors (nothing is launched): RMSNORM_E_DTYPE,
 * RMSNORM_E_SHAPE (tokens < 0, heads < 1, head_dim odd or outside [2, 1024],
 * heads * head_dim > 2^24, table_rows < 1, table_rows * head_dim / 2 > 2^28,
 * tokens > RMSNORM_M_MAX, token_stride * tokens beyond 2^60 elements,
 * seq_len outside [1, table_rows] without positions), RMSNORM_E_STRIDE
 * (token_stride < heads * head_dim), RMSNORM_E_NULL, RMSNORM_E_ALIGN,
 * RMSNORM_E_ALIAS (q overlaps a table or positions).
 */
#ifndef ROPE_H
#define ROPE_H

#include "rmsnorm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Forward rotation of q, in place. */
int rope_fwd(void* q, int64_t tokens, int64_t heads, int64_t head_dim, int64_t token_stride, const float* cos,
             const float* sin, int64_t table_rows, const int32_t* positions, int64_t seq_len, int dtype,
             hipStream_t stream);

/* Backward: the inverse rotation (sin negated) of the gradient dq, in place. */
int rope_bwd(void* dq, int64_t tokens, int64_t heads, int64_t head_dim, int64_t token_stride, const float* cos,
             const float* sin, int64_t table_rows, const int32_t* positions, int64_t seq_len, int dtype,
             hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ROPE_H */
