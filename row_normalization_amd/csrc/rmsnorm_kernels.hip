// gfx950 (CDNA4) kernels for fused RMSNorm forward and backward.
//
// What is computed (Triton RMSNorm tutorial "Hướng dẫn Triton RMSNorm:
// kernel, backward và…", partitech.com; Gemma weight from the Unsloth kernel
// walkthrough "02 · 手写 Triton kernel", section 3):
//   forward   r = 1/sqrt(mean(x^2) + eps) per row, y = x * r * w
//   backward  u = dy * w, dx = r*u - x * r^3 * mean(u*x), dgamma = sum_rows dy*x*r
// with w = gamma, or 1 + gamma for Gemma.
//
// How it maps to the hardware.  The work is a bandwidth-bound row reduction
// (about 1 flop per byte), so there is no MFMA: everything is about moving
// each byte of x, dy, y and dx through HBM exactly once.
//  - Each lane owns whole 16-byte column vectors of a row (8 bf16/fp16 or 4 fp32)
//    and issues all of its loads for the row before any arithmetic; a row is
//    read once and never re-read.
//  - Every row access is a raw buffer load/store through a per-row buffer
//    descriptor whose range is the row's bytes (zero for rows past M).  The
//    hardware range check turns the masked tail and missing rows into
//    zero-returning loads and dropped stores, so every access is one
//    unconditional instruction: no branches around memory operations, and
//    the compiler can count the operations in flight exactly (with
//    branch-guarded loads it has to wait for all of them, which serialises
//    the backward's row pipeline).
//  - Upcast to fp32 on load; sums in fp32; one rounding (RNE, the gfx950
//    packed bf16/fp16 converts) on store.
//  - Row sums are reduced inside the wave with DPP row operations, a
//    ds_swizzle across the 32-lane halves and two readlanes (no LDS traffic).
//    When a row spans several waves the per-wave sums meet in LDS behind one
//    barrier; the LDS slots are double-buffered by step parity so one barrier
//    per row suffices.
//  - The backward is a persistent grid: each workgroup owns a fixed set of
//    rows, keeps the weight and its dgamma column partials in registers
//    across them, and writes one fp32 partial row at the end (row groups of
//    the workgroup are combined in LDS in a fixed order).  Where one
//    workgroup fills its CU, it issues the next row's loads before working
//    on a row.  A second small kernel sums the partial rows per column in a
//    fixed order.  No atomics touch data, so every result is bitwise
//    reproducible.
//  - dx may be written over dy: each lane reads its own dy elements before it
//    writes the same elements of dx, and no other lane touches them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "rmsnorm.h"

namespace rmsn {
namespace {
using namespace dev;

// ---------------------------------------------------------------------------
// Cache policy of the streamed row operands: every byte of x, dy, y and dx is
// touched once per pass, so all of them use the nontemporal forms, which do
// not allocate in L2 or the 256 MB Infinity Cache.  Measured on MI355X at
// 16384 x 8192 bf16: an allocating x load in the forward loses a third of
// the forward's bandwidth when the cache holds dirty lines (each allocation
// then costs a write-back), and only pays off when the backward of the same
// rows runs right after the forward and finds x still cached.
// ---------------------------------------------------------------------------
constexpr int kFwdLoadX = kNontemporal;
constexpr int kFwdStoreY = kNontemporal;
constexpr int kBwdLoadXdy = kNontemporal;
constexpr int kBwdStoreDx = kNontemporal;

// ---------------------------------------------------------------------------
// Forward: y = x * r * w, rstd = r.
// The grid either covers the row groups (one step each; the hardware
// dispatcher balances the load) or, where that fills the compute units
// evenly, is persistent (a fixed number of workgroups per CU stepping
// through the rows).  gamma is loaded once per workgroup and kept packed in
// registers across its rows.
// ---------------------------------------------------------------------------
// One forward row's work once its x is in registers: r (written by one lane
// of the row group), then y.
template <typename S, int VEC, int ITERS>
__device__ __forceinline__ void fwd_row(Pack<S, VEC> (&xv)[ITERS], const Pack<S, VEC> (&gv)[ITERS], const FwdArgs& a,
                                        int64_t step, const Lane& L, float (*red)[kMaxBlockWaves], Rsrc rr,
                                        uint32_t voff, uint32_t iter_bytes, uint32_t row_bytes) {
  const int64_t row = row_of(step, a.row_iters, a.rpb, L.group);
  const bool active = row < a.M;
  S* y = static_cast<S*>(a.y);
  const Rsrc ry = make_rsrc(y + (active ? row * a.stride : 0), active ? row_bytes : 0u);

  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < ITERS; ++i)
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const float f = xv[i].get(e);
      ss = fmaf(f, f, ss);
    }
#pragma unroll
  for (int i = 0; i < ITERS; ++i) xv[i].keep_packed();
  ss = wave_sum(ss);
  if (a.wpr > 1) ss = group_sum(ss, red, step, L.wave, L.group, a.wpr, L.lane);

  // mean over the true N (not a padded width), eps under the root
  const float r = rsqrtf(fmaf(ss, a.inv_n, a.eps));
  // one lane per row writes r; every other lane's offset is out of range
  const bool writer = active && L.wv == 0 && L.lane == 0;
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, r), rr,
                                        writer ? static_cast<uint32_t>(row) * 4u : kOutOfRange, 0, kDefault);

#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    float o[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float normed = xv[i].get(e) * r;
      if (a.round_normed) normed = round_to<S>(normed);  // uniform branch
      o[e] = normed * (gv[i].get(e) + a.w_off);
    }
    buf_store<S, VEC, kFwdStoreY>(round_pack<S, VEC>(o), ry, voff + i * iter_bytes);
  }
}

template <typename S, int VEC, int ITERS, bool EARLY>
__global__ __launch_bounds__(1024) void rmsnorm_fwd_kernel(const FwdArgs a) {
  constexpr uint32_t kPack = Pack<S, VEC>::kBytes;
  const Lane L(a.wpr);
  __shared__ float red[2][kMaxBlockWaves];

  const uint32_t voff = L.first_vec() * kPack;
  const uint32_t iter_bytes = static_cast<uint32_t>(a.wpr) * kWave * kPack;
  const uint32_t row_bytes = static_cast<uint32_t>(a.N) * sizeof(S);
  const Rsrc rg = make_rsrc(a.gamma, row_bytes);
  const Rsrc rr = make_rsrc(a.rstd, static_cast<uint32_t>(a.M) * 4u);
  const S* x = static_cast<const S*>(a.x);

  // gamma once per workgroup (the same columns for every row it takes)
  Pack<S, VEC> gv[ITERS];
#pragma unroll
  for (int i = 0; i < ITERS; ++i) gv[i] = buf_load<S, VEC, kDefault>(rg, voff + i * iter_bytes);

  // row `step`'s x, all of this lane's loads before any arithmetic
  auto load_row = [&](Pack<S, VEC>(&xv)[ITERS], int64_t step) {
    const int64_t row = row_of(step, a.row_iters, a.rpb, L.group);
    const bool active = row < a.M;
    const Rsrc rx = make_rsrc(x + (active ? row * a.stride : 0), active ? row_bytes : 0u);
#pragma unroll
    for (int i = 0; i < ITERS; ++i) xv[i] = buf_load<S, VEC, kFwdLoadX>(rx, voff + i * iter_bytes);
  };

  Pack<S, VEC> xv[ITERS];
  if constexpr (EARLY) {
    // The first row's loads go out before anything waits for gamma: the
    // weight's unpacking, which the compiler hoists out of the row loop, then
    // waits for gamma alone with the row's loads in flight.  Each step then
    // loads the next row, if there is one, after storing its own (a load of a
    // row past the last step, even one that reads nothing, keeps a one-step
    // workgroup alive for its round trip).
    load_row(xv, 0);
    __builtin_amdgcn_sched_barrier(0);
    for (int64_t step = 0; step < a.row_iters; ++step) {
      fwd_row(xv, gv, a, step, L, red, rr, voff, iter_bytes, row_bytes);
      if (step + 1 < a.row_iters) load_row(xv, step + 1);
    }
  } else {
    // Load a row, then work on it.
    for (int64_t step = 0; step < a.row_iters; ++step) {
      load_row(xv, step);
      fwd_row(xv, gv, a, step, L, red, rr, voff, iter_bytes, row_bytes);
    }
  }
}

// ---------------------------------------------------------------------------
// Backward row pass: dx, and per-workgroup dgamma partial rows.
// Persistent: each workgroup takes a fixed set of rows.  A lane keeps, for
// the columns it owns, the weight w = gamma (+1 for Gemma) in fp32 and its
// dgamma partials in fp32 registers across all its rows.
// ---------------------------------------------------------------------------
template <typename S, int VEC, int ITERS>
struct BwdRow {
  Pack<S, VEC> x[ITERS];
  Pack<S, VEC> dy[ITERS];
  float r;
};

// Offsets and descriptors a backward lane uses for every row.
struct BwdGeom {
  uint32_t voff;        // byte offset of the lane's first vector in a row
  uint32_t iter_bytes;  // bytes between the lane's successive vectors
  uint32_t row_bytes;   // N * sizeof(S)
  Rsrc rstd;            // the M saved r values
};

template <typename S, int VEC, int ITERS>
__device__ __forceinline__ void bwd_load_row(BwdRow<S, VEC, ITERS>& t, const BwdArgs& a, int64_t step, const Lane& L,
                                             const BwdGeom& G) {
  const int64_t row = row_of(step, a.row_iters, a.rpb, L.group);
  const bool active = row < a.M;
  const int64_t off = active ? row * a.stride : 0;
  const Rsrc rx = make_rsrc(static_cast<const S*>(a.x) + off, active ? G.row_bytes : 0u);
  const Rsrc rd = make_rsrc(static_cast<const S*>(a.dy) + off, active ? G.row_bytes : 0u);
#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    t.x[i] = buf_load<S, VEC, kBwdLoadXdy>(rx, G.voff + i * G.iter_bytes);
    t.dy[i] = buf_load<S, VEC, kBwdLoadXdy>(rd, G.voff + i * G.iter_bytes);
  }
  // r of a missing row reads as zero (out of the descriptor's range)
  t.r = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                      G.rstd, active ? static_cast<uint32_t>(row) * 4u : kOutOfRange, 0, kDefault));
}

template <typename S, int VEC, int ITERS>
__device__ __forceinline__ void bwd_process_row(BwdRow<S, VEC, ITERS>& t, const BwdArgs& a, int64_t step,
                                                const float (&w)[ITERS][VEC], float (&acc)[ITERS][VEC],
                                                float (*red)[kMaxBlockWaves], const Lane& L, const BwdGeom& G) {
  const int64_t row = row_of(step, a.row_iters, a.rpb, L.group);
  const bool active = row < a.M;
  const int64_t off = active ? row * a.stride : 0;
  // dx may be the dy buffer itself; every element of dy this lane owns was
  // loaded into registers before this point
  const Rsrc rdx = make_rsrc(static_cast<S*>(a.dx) + off, active ? G.row_bytes : 0u);

  // sum over the row of u*x with u = dy*w
  float dot = 0.f;
#pragma unroll
  for (int i = 0; i < ITERS; ++i)
#pragma unroll
    for (int e = 0; e < VEC; ++e) dot = fmaf(t.dy[i].get(e) * w[i][e], t.x[i].get(e), dot);
#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    t.x[i].keep_packed();
    t.dy[i].keep_packed();
  }
  dot = wave_sum(dot);
  if (a.wpr > 1) dot = group_sum(dot, red, step, L.wave, L.group, a.wpr, L.lane);

  // dx = r*u - x * (r^3 * mean(u*x)), mean over the true N
  const float r = t.r;
  const float c = r * r * r * (dot * a.inv_n);
#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    float o[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const float xf = t.x[i].get(e);
      const float df = t.dy[i].get(e);
      o[e] = fmaf(-xf, c, r * (df * w[i][e]));
      acc[i][e] = fmaf(df * xf, r, acc[i][e]);  // dgamma contribution dy*x*r (zero past the row's end)
    }
    buf_store<S, VEC, kBwdStoreDx>(round_pack<S, VEC>(o), rdx, G.voff + i * G.iter_bytes);
  }
}

template <typename S, int VEC, int ITERS>
__global__ __launch_bounds__(1024) void rmsnorm_bwd_rows_kernel(const BwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) float comb[];  // N floats, when rpb > 1
  __shared__ float red[2][kMaxBlockWaves];
  constexpr uint32_t kPack = Pack<S, VEC>::kBytes;
  const Lane L(a.wpr);
  BwdGeom G;
  G.voff = static_cast<uint32_t>(L.template wave_vec<ITERS>(0)) * kPack;
  G.iter_bytes = static_cast<uint32_t>(kWave) * kPack;
  G.row_bytes = static_cast<uint32_t>(a.N) * sizeof(S);
  G.rstd = make_rsrc(a.rstd, static_cast<uint32_t>(a.M) * 4u);

  BwdRow<S, VEC, ITERS> ta;

  float w[ITERS][VEC];
  float acc[ITERS][VEC];
  {
    const Rsrc rg = make_rsrc(a.gamma, G.row_bytes);
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const Pack<S, VEC> g = buf_load<S, VEC, kDefault>(rg, G.voff + i * G.iter_bytes);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        w[i][e] = g.get(e) + a.w_off;
        acc[i][e] = 0.f;
      }
    }
  }

  bool pipelined = false;
  if constexpr (bwd_pipeline_fits(RowOp::kRmsBwd, dtype_code<S>(), VEC, ITERS)) pipelined = a.pipeline;
  if (pipelined) {
    // One workgroup per CU: the next row's loads are in flight during this
    // row's reduction, barrier and stores, so the memory system is not idle
    // while they run.  Rows are still processed in order (the LDS slots of
    // the row sums alternate by step).  Every load is unconditional: steps
    // past the last one hold only rows past M, whose loads read zero and
    // whose stores are dropped (and whose zero operands add nothing to the
    // partials), so the trip count can be even and the compiler sees the
    // same memory operations on every trip.  It then waits for exactly the
    // row it is about to use; a load under a condition made it wait for every
    // operation in flight, the next row's loads included.  The scheduling
    // barriers keep each row's arithmetic below the previous row's stores.
    BwdRow<S, VEC, ITERS> tb;
    bwd_load_row(ta, a, 0, L, G);
    __builtin_amdgcn_sched_barrier(0);
    for (int64_t step = 0; step < a.row_iters; step += 2) {
      bwd_load_row(tb, a, step + 1, L, G);
      __builtin_amdgcn_sched_barrier(0);
      bwd_process_row(ta, a, step, w, acc, red, L, G);
      bwd_load_row(ta, a, step + 2, L, G);
      __builtin_amdgcn_sched_barrier(0);
      bwd_process_row(tb, a, step + 1, w, acc, red, L, G);
    }
  } else {
    // One row at a time: with two workgroups per CU the other workgroup's
    // loads cover a row's reduction and barrier (pipelined, this pass ran
    // 2-8 % slower at 16384 x 8192 and 32768 x 5120).
    for (int64_t step = 0; step < a.row_iters; ++step) {
      bwd_load_row(ta, a, step, L, G);
      bwd_process_row(ta, a, step, w, acc, red, L, G);
    }
  }

  // One partial row per workgroup: row groups are added in LDS in group order.
  float* prow = a.partials + static_cast<int64_t>(blockIdx.x) * a.N;
  const Rsrc rp = make_rsrc(prow, static_cast<uint32_t>(a.N) * 4u);
  const uint32_t voff32 = static_cast<uint32_t>(L.template wave_vec<ITERS>(0)) * VEC * 4u;
  const uint32_t iter32 = static_cast<uint32_t>(kWave) * VEC * 4u;
  // The last row group adds the sum of the groups before it (left in LDS) to
  // its own and writes the partial row; every group covers every column, and
  // lanes past the row's end store out of the descriptor's range.
  for (int g = 0; g < a.rpb - 1; ++g) {
    if (g > 0) __syncthreads();
    if (L.group == g) {
#pragma unroll
      for (int i = 0; i < ITERS; ++i) {
        const int v = L.template wave_vec<ITERS>(i);
        if (v < a.nvec) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            float* cell = comb + v * VEC + e;
            *cell = (g == 0) ? acc[i][e] : *cell + acc[i][e];
          }
        }
      }
    }
  }
  if (a.rpb > 1) {
    __syncthreads();
    if (L.group != a.rpb - 1) return;
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const int v = L.template wave_vec<ITERS>(i);
      if (v < a.nvec) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[i][e] += comb[v * VEC + e];
      }
    }
  }
  if (a.partials_nt) {
#pragma unroll
    for (int i = 0; i < ITERS; ++i) buf_store_f32<VEC, kNontemporal>(acc[i], rp, voff32 + i * iter32);
  } else {
#pragma unroll
    for (int i = 0; i < ITERS; ++i) buf_store_f32<VEC, kDefault>(acc[i], rp, voff32 + i * iter32);
  }
}

// ---------------------------------------------------------------------------
// dgamma[j] = sum over partial rows p (in order) of partials[p, j].
// Block: kReduceCols column threads (VEC columns each) x kReduceSlices row
// slices; slice s sums rows s, s + slices, ...; the slices are then added in
// slice order.  Loads go through a descriptor over the whole partials table,
// so rows past the end read as zero and every load is unconditional.  They
// use the nontemporal policy: the partial rows are read once, and allocating
// them in the caches costs the next launch's operands their place there.
// Measured on MI355X (interleaved comparison, the kernel after the row pass
// that wrote the partials): RMSNorm headline step (16384 x 8192) 0.8 %,
// 8192 x 16384 backward 1.3 %, 4096 x 4096 1.4 %, LayerNorm fp16 backward at
// 4096 x 2048-12288 1.6-5.4 % and 1151 x 8192 5.1 % faster (4096 x 1024
// +0.9 %).  Launched back to back on its own, reading the same table again
// and again, it is slower with it (3.9 -> 4.5 us at 16384 x 8192), a case
// training does not have.
// blockIdx.y picks the table when two are reduced in one launch (the
// LayerNorm weight and bias gradients).
// ---------------------------------------------------------------------------
template <int VEC>
__global__ __launch_bounds__(kReduceCols * kReduceSlices) void rmsnorm_dgamma_reduce_kernel(const ReduceArgs a) {
  constexpr int kUnroll = 16;
  __shared__ float part[kReduceSlices][kReduceCols * VEC];
  const int tc = threadIdx.x % kReduceCols;
  const int ts = threadIdx.x / kReduceCols;
  const int col = (blockIdx.x * kReduceCols + tc) * VEC;
  const float* table = a.partials + static_cast<int64_t>(blockIdx.y) * a.rows * a.N;
  float* out = blockIdx.y ? a.dgamma2 : a.dgamma;
  const Rsrc rp = make_rsrc(table, static_cast<uint32_t>(a.rows * a.N) * 4u);
  const uint32_t slice_bytes = static_cast<uint32_t>(kReduceSlices) * static_cast<uint32_t>(a.N) * 4u;
  const uint32_t voff = (static_cast<uint32_t>(ts) * static_cast<uint32_t>(a.N) + static_cast<uint32_t>(col)) * 4u;
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  const int64_t trips = (a.rows + kReduceSlices - 1) / kReduceSlices;
  for (int64_t k = 0; k < trips; k += kUnroll) {
    Pack<float, VEC> v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      v[u] = buf_load<float, VEC, kNontemporal>(rp, voff + static_cast<uint32_t>(k + u) * slice_bytes);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] += v[u].get(e);
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) part[ts][tc * VEC + e] = acc[e];
  __syncthreads();
  if (ts == 0 && col < a.N) {
    float o[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float t = part[0][tc * VEC + e];
      for (int s = 1; s < kReduceSlices; ++s) t += part[s][tc * VEC + e];
      o[e] = t;
    }
    *reinterpret_cast<Pack<float, VEC>*>(out + col) = round_pack<float, VEC>(o);
  }
}

// ---------------------------------------------------------------------------
// Host-side dispatch to the compiled instantiations.
// ---------------------------------------------------------------------------
template <typename S, int VEC, int ITERS>
hipError_t fwd_inst(const RowPlan& p, const FwdArgs& a, hipStream_t s) {
  if constexpr (VEC * ITERS > lane_elems_cap(RowOp::kRmsFwd, sizeof(S))) {
    return hipErrorInvalidValue;  // beyond the register model: never planned, not compiled
  } else {
    // The first row's loads ahead of the weight's unpacking: compiled for
    // 16-byte vectors and at most 8 per lane (with 16 the early row's
    // registers spill), and launched where the plan asks for it.
    if constexpr (VEC * sizeof(S) == 16 && ITERS <= 8) {
      if (a.first_row_early) {
        hipLaunchKernelGGL((rmsnorm_fwd_kernel<S, VEC, ITERS, true>), dim3(static_cast<unsigned>(p.grid)),
                           dim3(p.threads()), 0, s, a);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((rmsnorm_fwd_kernel<S, VEC, ITERS, false>), dim3(static_cast<unsigned>(p.grid)),
                       dim3(p.threads()), 0, s, a);
    return hipGetLastError();
  }
}

template <typename S, int VEC, int ITERS>
hipError_t bwd_inst(const RowPlan& p, const BwdArgs& a, hipStream_t s) {
  if constexpr (VEC * ITERS > lane_elems_cap(RowOp::kRmsBwd, sizeof(S))) {
    return hipErrorInvalidValue;  // beyond the register model: never planned, not compiled
  } else {
    const size_t lds = p.rpb > 1 ? static_cast<size_t>(a.N) * sizeof(float) : 0;
    hipLaunchKernelGGL((rmsnorm_bwd_rows_kernel<S, VEC, ITERS>), dim3(static_cast<unsigned>(p.grid)),
                       dim3(p.threads()), lds, s, a);
    return hipGetLastError();
  }
}

template <typename S, int VEC>
hipError_t fwd_vec(const RowPlan& p, const FwdArgs& a, hipStream_t s) {
  return pick_iters<FwdArgs, fwd_inst<S, VEC, 1>, fwd_inst<S, VEC, 2>, fwd_inst<S, VEC, 4>, fwd_inst<S, VEC, 5>,
                    fwd_inst<S, VEC, 8>, fwd_inst<S, VEC, 16>>(p, a, s);
}

template <typename S, int VEC>
hipError_t bwd_vec(const RowPlan& p, const BwdArgs& a, hipStream_t s) {
  return pick_iters<BwdArgs, bwd_inst<S, VEC, 1>, bwd_inst<S, VEC, 2>, bwd_inst<S, VEC, 4>, bwd_inst<S, VEC, 5>,
                    bwd_inst<S, VEC, 8>, bwd_inst<S, VEC, 16>>(p, a, s);
}

}  // namespace

hipError_t launch_fwd(int dtype, const RowPlan& p, const FwdArgs& a, hipStream_t s) {
  if (dtype == 0) {
    switch (p.vec) {
      case 1: return fwd_vec<float, 1>(p, a, s);
      case 2: return fwd_vec<float, 2>(p, a, s);
      case 4: return fwd_vec<float, 4>(p, a, s);
    }
  } else if (dtype == 1) {
    switch (p.vec) {
      case 1: return fwd_vec<uint16_t, 1>(p, a, s);
      case 2: return fwd_vec<uint16_t, 2>(p, a, s);
      case 4: return fwd_vec<uint16_t, 4>(p, a, s);
      case 8: return fwd_vec<uint16_t, 8>(p, a, s);
    }
  } else if (dtype == 2) {
    switch (p.vec) {
      case 1: return fwd_vec<_Float16, 1>(p, a, s);
      case 2: return fwd_vec<_Float16, 2>(p, a, s);
      case 4: return fwd_vec<_Float16, 4>(p, a, s);
      case 8: return fwd_vec<_Float16, 8>(p, a, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_rows(int dtype, const RowPlan& p, const BwdArgs& a, hipStream_t s) {
  if (dtype == 0) {
    switch (p.vec) {
      case 1: return bwd_vec<float, 1>(p, a, s);
      case 2: return bwd_vec<float, 2>(p, a, s);
      case 4: return bwd_vec<float, 4>(p, a, s);
    }
  } else if (dtype == 1) {
    switch (p.vec) {
      case 1: return bwd_vec<uint16_t, 1>(p, a, s);
      case 2: return bwd_vec<uint16_t, 2>(p, a, s);
      case 4: return bwd_vec<uint16_t, 4>(p, a, s);
      case 8: return bwd_vec<uint16_t, 8>(p, a, s);
    }
  } else if (dtype == 2) {
    switch (p.vec) {
      case 1: return bwd_vec<_Float16, 1>(p, a, s);
      case 2: return bwd_vec<_Float16, 2>(p, a, s);
      case 4: return bwd_vec<_Float16, 4>(p, a, s);
      case 8: return bwd_vec<_Float16, 8>(p, a, s);
    }
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Static scratch of rmsnorm_bwd_noalloc: the fp32 partial rows of the weight
// gradient, for callers that cannot allocate.  Every GPU the library runs on
// holds its own copy until the process ends.  On the host the name is only a
// stand-in for the symbol (passing it to a kernel would hand the kernel a
// host address): host code uses the device address that hipGetSymbolAddress
// returns for the current device, looked up once per device.
// ---------------------------------------------------------------------------
static __device__ __align__(256) float scratch[RMSNORM_STATIC_SCRATCH_BYTES / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_dgamma_reduce(int vec, int tables, const ReduceArgs& a, hipStream_t s) {
  const int cols = kReduceCols * vec;
  const dim3 grid(static_cast<unsigned>((a.N + cols - 1) / cols), static_cast<unsigned>(tables));
  if (tables != 1 && tables != 2) return hipErrorInvalidValue;
  if (vec == 4) {
    hipLaunchKernelGGL(rmsnorm_dgamma_reduce_kernel<4>, grid, dim3(kReduceCols * kReduceSlices), 0, s, a);
  } else if (vec == 1) {
    hipLaunchKernelGGL(rmsnorm_dgamma_reduce_kernel<1>, grid, dim3(kReduceCols * kReduceSlices), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rmsn
