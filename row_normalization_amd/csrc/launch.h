// Internal interface between the host-side C ABIs (rmsnorm_api.cpp and
// layernorm_api.cpp: argument validation and launch planning, no device code)
// and the gfx950 kernels (rmsnorm_kernels.hip, layernorm_kernels.hip).  Not
// installed, not part of the ABI.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace rmsn {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kMaxBlockWaves = 16; // 1024-thread workgroups at most

// A row kernel processes rows in "row groups": `wpr` waves cooperate on one
// row, `rpb` row groups share a workgroup (block = 64 * wpr * rpb threads).
// Lane `l` of wave `w` in a group owns the VEC-element column vectors
// v = (i * wpr + w) * 64 + l for i < iters (the RMSNorm backward:
// v = (w * iters + i) * 64 + l); vectors at or past N / VEC are masked.  Rows are assigned statically: at step k, group g of block b takes
// row (k * grid + b) * rpb + g, for k < row_iters.
struct RowPlan {
  int vec;        // elements per vector load (16 bytes when alignment allows)
  int iters;      // vectors per lane (a compiled-in register-array length)
  int wpr;        // waves per row
  int rpb;        // row groups per block
  int64_t grid;   // workgroups
  int64_t row_iters;
  bool wide;      // LayerNorm's wide kernels (iters = 1024-vector chunks per row)
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
  int32_t first_row_early;  // host side: launch the build that issues the first row's loads before
                            // unpacking the weight (fwd_first_row_early)
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
  int32_t pipeline;     // 1: keep the next row's loads in flight during a row's work
  int32_t partials_nt;  // 1: write the partial rows with the nontemporal policy (partials_nontemporal)
};

// Column sums of one or two [rows, N] fp32 tables stored back to back
// (table t starts at partials + t * rows * N and is summed into dgamma for
// t = 0, into dgamma2 for t = 1).
struct ReduceArgs {
  const float* partials;
  float* dgamma;
  int64_t rows;
  int32_t N;
  float* dgamma2;  // null for one table
};

// LayerNorm forward: y = (x - mean) * rstd * weight + bias, mean and rstd per row.
struct LnFwdArgs {
  const void* x;
  const void* weight;
  const void* bias;
  void* y;
  float* mean;
  float* rstd;
  int64_t M;
  int64_t stride;
  int32_t N;
  int32_t nvec;
  float eps;
  float inv_n;
  int32_t wpr;
  int32_t rpb;
  int64_t row_iters;
  int32_t chunks;  // wide rows only: 1024-vector chunks per row
};

// LayerNorm backward row pass: dx, and per-workgroup partial rows of dw
// (partials[0 .. grid)) and db (partials[grid .. 2 grid)).
struct LnBwdArgs {
  const void* x;
  const void* weight;
  const void* dy;
  const float* mean;
  const float* rstd;
  void* dx;  // may equal dy
  float* partials;  // [2, grid, N] fp32
  int64_t M;
  int64_t stride;
  int32_t N;
  int32_t nvec;
  float inv_n;
  int32_t wpr;
  int32_t rpb;
  int64_t row_iters;
  int32_t pipeline;     // as in BwdArgs
  int32_t partials_nt;  // as in BwdArgs
  int32_t chunks;       // wide rows only: 1024-vector chunks per row
};

// LayerNorm rows of 16-bit elements beyond the register plans (up to
// kLnWideMaxN elements, 64 KB) run in the wide kernels: one 1024-thread
// workgroup per row, lane t owning vector k * 1024 + t of each 1024-vector
// chunk k, so at most kLnWideColsPerLane columns per lane.
constexpr int kLnWideMaxN = 32768;
constexpr int kLnWideColsPerLane = kLnWideMaxN / 1024;
// The wide backward over 16-byte vectors is compiled for rows of
// kLnWideHeldChunksMin..kLnWideHeldChunksMax chunks (8192 elements each) and
// keeps the weight row in LDS, chunks * 16 KB of it: within gfx950's 160 KB
// of LDS per workgroup (kLdsPerWorkgroup), beside its 256-byte sum table.
constexpr int kLdsPerWorkgroup = 160 * 1024;
constexpr int kLnWideHeldChunksMin = 3;  // rows beyond the register plans' 16384 elements
constexpr int kLnWideHeldChunksMax = kLnWideMaxN / 8192;
constexpr int kLnWideHeldLdsBytes(int chunks) { return chunks * 1024 * 16; }
static_assert(kLnWideHeldLdsBytes(kLnWideHeldChunksMax) + 256 <= kLdsPerWorkgroup, "weight row fits LDS");

// RoPE: one work item = one token, one group of kRopeGroup heads, one VEC
// vector of the half-head (and the matching vector of the other half).
constexpr int kRopeGroup = 4;
constexpr int kEltThreads = 256;  // workgroup size of the elementwise kernels
struct RopeArgs {
  void* q;
  const float* cos;
  const float* sin;
  const int32_t* positions;  // null: t mod seq_len
  int64_t tokens;
  int64_t stride;      // elements between tokens
  int64_t table_rows;
  int64_t seq_len;
  int64_t items;       // tokens * groups * nvh
  int32_t heads;
  int32_t half;        // head_dim / 2
  int32_t groups;      // ceil(heads / kRopeGroup)
  int32_t nvh;         // half / VEC
  float sin_sign;      // +1 forward, -1 backward
};

// SwiGLU over [M, N] with one row stride; workgroup b (grid-stride) takes row
// b / tiles and column tile b mod tiles of kSwigluUnroll * kEltThreads vectors.
// Dense operands (row stride == N) are walked as one flat array cut into rows
// of kSwigluFlatRow elements (a whole number of tiles), so only the very last
// tile can be partly empty; last_row_elems is the length of the last row.
constexpr int kSwigluUnroll = 2;
constexpr int64_t kSwigluFlatRow = 65536;
struct SwigluArgs {
  const void* e;
  const void* g;
  const void* dh;  // backward only
  void* h;
  void* df;        // backward only
  void* de;        // backward only
  int64_t M;
  int64_t stride;
  int64_t blocks;  // M * tiles
  int64_t last_row_elems;
  int32_t N;
  int32_t tiles;
};

// Compiled-in register-array lengths for the row kernels.
constexpr int kItersSet[] = {1, 2, 4, 5, 8, 16};
constexpr int kItersMax = 16;

// Register model of the row kernels: the elements of a row one lane may own
// (vec * iters at most) so that its row data fits in kLaneDataRegs 32-bit
// registers (of the 128 a lane of a 1024-thread workgroup may use).  Costs
// per element, in quarter registers: a packed operand costs its element size,
// an fp32 value 4.
//   RMSNorm forward   x and gamma packed
//   RMSNorm backward  x and dy packed; fp32 weight and dgamma partial
//   LayerNorm forward x, weight and bias packed, plus a quarter register per
//                     element for the conversions of three operands (at 64
//                     fp16 elements per lane the compiler spills otherwise)
//   LayerNorm backward x and dy packed; fp32 weight, dw and db partials
// The host planner never picks more; the dispatch compiles nothing beyond it.
constexpr int kLaneDataRegs = 96;
enum class RowOp { kRmsFwd, kRmsBwd, kLnFwd, kLnBwd };
constexpr int lane_elems_cap(RowOp op, int elsize) {
  return kLaneDataRegs * 4 / (op == RowOp::kRmsFwd   ? 2 * elsize
                              : op == RowOp::kRmsBwd ? 2 * elsize + 8
                              : op == RowOp::kLnFwd  ? 3 * elsize + 1
                                                     : 2 * elsize + 12);
}

// The backwards' pipelined row loop keeps a second row's x and dy in
// registers.  It is compiled, and chosen, only where a lane holds at most
// two full 16-byte vectors of each operand (beyond that, or with narrower
// vectors and so more loads and offsets per row, the second row would
// spill), and for the bf16 LayerNorm backward only in its build for
// workgroups of at most kNarrowThreads threads: its third per-column table
// (the db partials) and bf16's unpacking take ~140 registers with two rows
// in flight, past the 128 a lane of a 1024-thread workgroup has, within the
// 256 of a 512-thread one (two waves per SIMD).  `max_threads` is the
// workgroup size the build is bounded to.
constexpr int kPipelineLaneVectors = 2;
constexpr int kNarrowThreads = 512;
constexpr bool bwd_pipeline_fits(RowOp op, int dtype, int vec, int iters, int max_threads = 1024) {
  return vec * (dtype == 0 ? 4 : 2) == 16 && iters <= kPipelineLaneVectors &&
         !(op == RowOp::kLnBwd && dtype == 1 && max_threads > kNarrowThreads);
}
// Whether a pipelined plan needs the build bounded to kNarrowThreads-thread
// workgroups (the bf16 LayerNorm backward).
constexpr bool bwd_needs_narrow_build(RowOp op, int dtype, int vec, int iters) {
  return !bwd_pipeline_fits(op, dtype, vec, iters) && bwd_pipeline_fits(op, dtype, vec, iters, kNarrowThreads);
}

// Tile of the dgamma reduction: kReduceCols column threads (a 128-byte row
// segment with 16-byte loads) x kReduceSlices row slices per 256-thread block.
constexpr int kReduceCols = 8;
constexpr int kReduceSlices = 32;

// dtype codes match rmsnorm_dtype (0 fp32, 1 bf16, 2 fp16).  Each returns hipSuccess or the launch error.
hipError_t launch_fwd(int dtype, const RowPlan& p, const FwdArgs& a, hipStream_t s);
hipError_t launch_bwd_rows(int dtype, const RowPlan& p, const BwdArgs& a, hipStream_t s);
// `tables` is 1 (dgamma) or 2 (dgamma and dgamma2).
hipError_t launch_dgamma_reduce(int vec, int tables, const ReduceArgs& a, hipStream_t s);
hipError_t launch_ln_fwd(int dtype, const RowPlan& p, const LnFwdArgs& a, hipStream_t s);
hipError_t launch_ln_bwd_rows(int dtype, const RowPlan& p, const LnBwdArgs& a, hipStream_t s);
// Wide LayerNorm rows (16-bit dtypes only): p.vec, p.grid, p.row_iters and
// a.chunks from plan_ln_wide.
hipError_t launch_ln_fwd_wide(int dtype, const RowPlan& p, const LnFwdArgs& a, hipStream_t s);
hipError_t launch_ln_bwd_wide(int dtype, const RowPlan& p, const LnBwdArgs& a, hipStream_t s);
hipError_t launch_rope(int dtype, int vec, const RopeArgs& a, hipStream_t s);
hipError_t launch_swiglu_fwd(int dtype, int vec, const SwigluArgs& a, hipStream_t s);
hipError_t launch_swiglu_bwd(int dtype, int vec, const SwigluArgs& a, hipStream_t s);

// The current device's copy of the library's static scratch (the fp32
// partial rows of rmsnorm_bwd_noalloc, RMSNORM_STATIC_SCRATCH_BYTES per GPU): its
// device address, looked up once per device.  Returns the lookup's error.
hipError_t static_scratch(void** ptr);

}  // namespace rmsn
