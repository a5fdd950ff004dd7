// Internal interface between the host-side C ABI (rmsnorm_api.cpp: argument
// validation and launch planning, no device code) and the gfx950 kernels
// (rmsnorm_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace rmsn {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kMaxBlockWaves = 16; // 1024-thread workgroups at most

// A row kernel processes rows in "row groups": `wpr` waves cooperate on one
// row, `rpb` row groups share a workgroup (block = 64 * wpr * rpb threads).
// Lane `l` of wave `w` in a group owns the VEC-element column vectors
// v = (i * wpr + w) * 64 + l for i < iters; vectors at or past N / VEC are
// masked.  Rows are assigned statically: at step k, group g of block b takes
// row (k * grid + b) * rpb + g, for k < row_iters.
struct RowPlan {
  int vec;        // elements per vector load (16 bytes when alignment allows)
  int iters;      // vectors per lane (a compiled-in register-array length)
  int wpr;        // waves per row
  int rpb;        // row groups per block
  int64_t grid;   // workgroups
  int64_t row_iters;
  int threads() const { return kWave * wpr * rpb; }
};

struct FwdArgs {
  const void* x;
  const void* gamma;
  void* y;
  float* rstd;
  int64_t M;
  int64_t stride;
  int32_t N;
  int32_t nvec;
  float eps;
  float inv_n;  // 1/N rounded to fp32
  float w_off;  // 0 (w = gamma) or 1 (Gemma: w = 1 + gamma)
  int32_t wpr;
  int32_t rpb;
  int64_t row_iters;
  int32_t round_normed;  // 1: round x*r to the I/O type before the weight multiply
};

struct BwdArgs {
  const void* x;
  const void* gamma;
  const void* dy;
  const float* rstd;
  void* dx;  // may equal dy
  float* partials;  // [grid, N] fp32
  int64_t M;
  int64_t stride;
  int32_t N;
  int32_t nvec;
  float inv_n;
  float w_off;
  int32_t wpr;
  int32_t rpb;
  int64_t row_iters;
};

struct ReduceArgs {
  const float* partials;
  float* dgamma;
  int64_t rows;
  int32_t N;
};

// Compiled-in register-array lengths for the row kernels.
constexpr int kItersSet[] = {1, 2, 4, 5, 8, 16};
constexpr int kItersMax = 16;

// Tile of the dgamma reduction: kReduceCols column threads (a 128-byte row
// segment with 16-byte loads) x kReduceSlices row slices per 256-thread block.
constexpr int kReduceCols = 8;
constexpr int kReduceSlices = 32;

// dtype codes match rmsnorm_dtype (0 fp32, 1 bf16, 2 fp16).  Each returns hipSuccess or the launch error.
hipError_t launch_fwd(int dtype, const RowPlan& p, const FwdArgs& a, hipStream_t s);
hipError_t launch_bwd_rows(int dtype, const RowPlan& p, const BwdArgs& a, hipStream_t s);
hipError_t launch_dgamma_reduce(int vec, const ReduceArgs& a, hipStream_t s);

}  // namespace rmsn
