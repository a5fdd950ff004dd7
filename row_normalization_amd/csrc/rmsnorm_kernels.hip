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
//  - Each lane owns whole 16-byte column vectors of a row (8 bf16 or 4 fp32)
//    and issues all of its loads for the row before any arithmetic, so a
//    wave has the whole row (or its share of it) in flight at once; a row is
//    read once and never re-read.
//  - Upcast to fp32 on load; sums in fp32; one rounding (RNE, the gfx950
//    packed bf16 convert) on store.
//  - Row sums are reduced inside the wave with DPP row operations, a
//    ds_swizzle across the 32-lane halves and two readlanes (no LDS traffic).
//    When a row spans several waves the per-wave sums meet in LDS behind one
//    barrier; the LDS slots are double-buffered by step parity so one barrier
//    per row suffices.
//  - The backward is a persistent grid: each workgroup owns a fixed set of
//    rows, keeps gamma and its dgamma column partials in registers across
//    them, and writes one fp32 partial row at the end (row groups of the
//    workgroup are combined in LDS in a fixed order).  A second small kernel
//    sums the partial rows per column in a fixed order.  No atomics touch
//    data, so every result is bitwise reproducible.
//  - dx may be written over dy: each lane reads its own dy elements before it
//    writes the same elements of dx, and no other lane touches them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "launch.h"

namespace rmsn {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// VEC consecutive elements with the storage type S (float, or uint16_t for
// bf16 bits), aligned to their full width so one load/store moves them.  They
// are held as 32-bit words (two bf16 per word) whenever the pack is at least
// 4 bytes wide.
template <typename S, int VEC>
struct alignas(sizeof(S) * VEC) Pack {
  static constexpr int kBytes = int(sizeof(S)) * VEC;
  static constexpr int kWords = kBytes >= 4 ? kBytes / 4 : 1;
  typedef typename std::conditional<(kBytes >= 4), uint32_t, uint16_t>::type Word;
  Word w[kWords];

  // element e as fp32 (bf16 -> fp32 is exact: the bits move to the top half)
  __device__ __forceinline__ float get(int e) const {
    if constexpr (sizeof(S) == 4) {
      return __builtin_bit_cast(float, w[e]);
    } else if constexpr (kBytes == 2) {
      return __builtin_bit_cast(float, static_cast<uint32_t>(w[0]) << 16);
    } else {
      const uint32_t word = w[e >> 1];
      return __builtin_bit_cast(float, (e & 1) ? (word & 0xFFFF0000u) : (word << 16));
    }
  }

  // Makes the compiler treat the words as changed here, so it re-derives the
  // fp32 values from the packed words after this point instead of keeping a
  // second, unpacked copy of the row alive across the row reduction (which
  // would double the registers a lane needs).  Emits no instruction.
  __device__ __forceinline__ void keep_packed() {
#pragma unroll
    for (int k = 0; k < kWords; ++k) {
      if constexpr (sizeof(Word) == 4) {
        asm volatile("" : "+v"(w[k]));
      } else {
        uint32_t t = w[k];
        asm volatile("" : "+v"(t));
        w[k] = static_cast<Word>(t);
      }
    }
  }
};

template <int VEC>
__device__ __forceinline__ void store_f32(float* dst, const float (&o)[VEC]) {
  Pack<float, VEC> p;
#pragma unroll
  for (int e = 0; e < VEC; ++e) p.w[e] = __builtin_bit_cast(uint32_t, o[e]);
  *reinterpret_cast<Pack<float, VEC>*>(dst) = p;
}

// Round VEC fp32 values once (to nearest even) to the storage type and store.
template <int VEC>
__device__ __forceinline__ void store_out(float* dst, const float (&o)[VEC]) {
  store_f32<VEC>(dst, o);
}
template <int VEC>
__device__ __forceinline__ void store_out(uint16_t* dst, const float (&o)[VEC]) {
  Pack<uint16_t, VEC> p;
  if constexpr (VEC == 1) {
    p.w[0] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(o[0]));
  } else {
#pragma unroll
    for (int e = 0; e < VEC; e += 2) {
      const f32x2_t f = {o[e], o[e + 1]};
      p.w[e >> 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
    }
  }
  *reinterpret_cast<Pack<uint16_t, VEC>*>(dst) = p;
}

template <typename S, int VEC>
__device__ __forceinline__ Pack<S, VEC> load_pack(const S* src) {
  return *reinterpret_cast<const Pack<S, VEC>*>(src);
}

template <typename S, int VEC>
__device__ __forceinline__ Pack<S, VEC> zero_pack() {
  Pack<S, VEC> p;
#pragma unroll
  for (int k = 0; k < Pack<S, VEC>::kWords; ++k) p.w[k] = 0;
  return p;
}

// v from another lane of the same 16-lane DPP row, selected by CTRL.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes of a wave; every lane receives the same total.
// quad_perm swaps (xor 1, xor 2), row_half_mirror and row_mirror complete
// the 16-lane rows, a ds_swizzle swaps 16-lane rows inside each 32-lane
// half, and the two halves are added through scalar readlanes.  The order of
// the additions is fixed, so the result is deterministic.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_move<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_move<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_move<0x141>(v);  // row_half_mirror
  v += dpp_move<0x140>(v);  // row_mirror
  v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));  // lane ^ 16
  const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  return lo + hi;
}

// Sum of one value per wave over the `wpr` waves of a row group, through LDS.
// Every wave of the group reads the slots in the same order.
__device__ __forceinline__ float group_sum(float wave_total, float (*red)[kMaxBlockWaves], int64_t step, int wave,
                                          int group, int wpr, int lane) {
  float* slot = red[step & 1];
  if (lane == 0) slot[wave] = wave_total;
  __syncthreads();
  float t = 0.f;
  for (int k = 0; k < wpr; ++k) t += slot[group * wpr + k];
  return t;
}

// ---------------------------------------------------------------------------
// Forward: y = x * r * w, rstd = r.
// One step per row group: the grid covers the rows (capped, then looped), so
// the hardware dispatcher balances the load.  gamma is read per row from the
// caches (it is N elements, shared by every row).
// ---------------------------------------------------------------------------
template <typename S, int VEC, int ITERS>
__global__ __launch_bounds__(1024) void rmsnorm_fwd_kernel(const FwdArgs a) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int group = wave / a.wpr;
  const int wv = wave - group * a.wpr;
  __shared__ float red[2][kMaxBlockWaves];

  const S* __restrict__ x = static_cast<const S*>(a.x);
  const S* __restrict__ gamma = static_cast<const S*>(a.gamma);
  S* __restrict__ y = static_cast<S*>(a.y);

  for (int64_t step = 0; step < a.row_iters; ++step) {
    const int64_t row = (step * gridDim.x + blockIdx.x) * a.rpb + group;
    const bool active = row < a.M;
    const int64_t off = active ? row * a.stride : 0;

    // all of this lane's loads for the row first: x, then gamma
    Pack<S, VEC> xv[ITERS];
    Pack<S, VEC> gv[ITERS];
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const int v = (i * a.wpr + wv) * kWave + lane;
      xv[i] = (active && v < a.nvec) ? load_pack<S, VEC>(x + off + static_cast<int64_t>(v) * VEC) : zero_pack<S, VEC>();
    }
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const int v = (i * a.wpr + wv) * kWave + lane;
      gv[i] = (active && v < a.nvec) ? load_pack<S, VEC>(gamma + v * VEC) : zero_pack<S, VEC>();
    }

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
    if (a.wpr > 1) ss = group_sum(ss, red, step, wave, group, a.wpr, lane);

    // mean over the true N (not a padded width), eps under the root
    const float r = rsqrtf(fmaf(ss, a.inv_n, a.eps));
    if (active && wv == 0 && lane == 0) a.rstd[row] = r;

#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const int v = (i * a.wpr + wv) * kWave + lane;
      if (active && v < a.nvec) {
        float o[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] = (xv[i].get(e) * r) * (gv[i].get(e) + a.w_off);
        store_out<VEC>(y + off + static_cast<int64_t>(v) * VEC, o);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Backward row pass: dx, and per-workgroup dgamma partial rows.
// Persistent: each workgroup takes a fixed set of rows.  The weight
// w = gamma (+1 for Gemma) is converted to fp32 once per workgroup into LDS;
// the dgamma partials of a lane's columns live in registers across all its
// rows.
// ---------------------------------------------------------------------------
template <typename S, int VEC, int ITERS>
__global__ __launch_bounds__(1024) void rmsnorm_bwd_rows_kernel(const BwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) float lds_w[];  // N floats: w, later reused to combine the partial rows
  __shared__ float red[2][kMaxBlockWaves];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int group = wave / a.wpr;
  const int wv = wave - group * a.wpr;

  const S* __restrict__ x = static_cast<const S*>(a.x);
  const S* __restrict__ gamma = static_cast<const S*>(a.gamma);
  const float* __restrict__ rstd = a.rstd;
  // dy and dx may be the same buffer: no __restrict__ on either.
  const S* dy = static_cast<const S*>(a.dy);
  S* dx = static_cast<S*>(a.dx);

  for (int c = tid; c < a.N; c += blockDim.x) {
    const Pack<S, 1> g = load_pack<S, 1>(gamma + c);
    lds_w[c] = g.get(0) + a.w_off;
  }
  __syncthreads();

  float acc[ITERS][VEC];
#pragma unroll
  for (int i = 0; i < ITERS; ++i)
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[i][e] = 0.f;

  for (int64_t step = 0; step < a.row_iters; ++step) {
    const int64_t row = (step * gridDim.x + blockIdx.x) * a.rpb + group;
    const bool active = row < a.M;
    const int64_t off = active ? row * a.stride : 0;

    Pack<S, VEC> xv[ITERS];
    Pack<S, VEC> dv[ITERS];
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const int v = (i * a.wpr + wv) * kWave + lane;
      const bool ok = active && v < a.nvec;
      xv[i] = ok ? load_pack<S, VEC>(x + off + static_cast<int64_t>(v) * VEC) : zero_pack<S, VEC>();
      dv[i] = ok ? load_pack<S, VEC>(dy + off + static_cast<int64_t>(v) * VEC) : zero_pack<S, VEC>();
    }
    const float r = active ? rstd[row] : 0.f;

    // sum over the row of u*x with u = dy*w
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const int v = (i * a.wpr + wv) * kWave + lane;
      const Pack<float, VEC> w = load_pack<float, VEC>(lds_w + (v < a.nvec ? v : 0) * VEC);
#pragma unroll
      for (int e = 0; e < VEC; ++e) dot = fmaf(dv[i].get(e) * w.get(e), xv[i].get(e), dot);
    }
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      xv[i].keep_packed();
      dv[i].keep_packed();
    }
    dot = wave_sum(dot);
    if (a.wpr > 1) dot = group_sum(dot, red, step, wave, group, a.wpr, lane);

    // dx = r*u - x * (r^3 * mean(u*x)), mean over the true N
    const float c = r * r * r * (dot * a.inv_n);
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const int v = (i * a.wpr + wv) * kWave + lane;
      if (active && v < a.nvec) {
        const Pack<float, VEC> w = load_pack<float, VEC>(lds_w + v * VEC);
        float o[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float xf = xv[i].get(e);
          const float df = dv[i].get(e);
          o[e] = fmaf(-xf, c, r * (df * w.get(e)));
          acc[i][e] = fmaf(df * xf, r, acc[i][e]);  // dgamma contribution dy*x*r
        }
        store_out<VEC>(dx + off + static_cast<int64_t>(v) * VEC, o);
      }
    }
  }

  // One partial row per workgroup: row groups are added in LDS in group order.
  float* prow = a.partials + static_cast<int64_t>(blockIdx.x) * a.N;
  if (a.rpb == 1) {
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const int v = (i * a.wpr + wv) * kWave + lane;
      if (v < a.nvec) store_f32<VEC>(prow + v * VEC, acc[i]);
    }
    return;
  }
  float* comb = lds_w;  // w is no longer needed once every wave passes the next barrier
  for (int g = 0; g < a.rpb; ++g) {
    __syncthreads();
    if (group == g) {
#pragma unroll
      for (int i = 0; i < ITERS; ++i) {
        const int v = (i * a.wpr + wv) * kWave + lane;
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
  __syncthreads();
  for (int col = tid; col < a.N; col += blockDim.x) prow[col] = comb[col];
}


// ---------------------------------------------------------------------------
// dgamma[j] = sum over partial rows p (in order) of partials[p, j].
// Block: kReduceCols column threads (VEC columns each) x kReduceSlices row
// slices; slice s sums rows s, s + slices, ...; the slices are then added in
// slice order.
// ---------------------------------------------------------------------------
template <int VEC>
__global__ __launch_bounds__(kReduceCols * kReduceSlices) void rmsnorm_dgamma_reduce_kernel(const ReduceArgs a) {
  __shared__ float part[kReduceSlices][kReduceCols * VEC];
  const int tc = threadIdx.x % kReduceCols;
  const int ts = threadIdx.x / kReduceCols;
  const int col = (blockIdx.x * kReduceCols + tc) * VEC;
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  if (col < a.N) {
    const float* __restrict__ p = a.partials + col;
#pragma unroll 8
    for (int64_t row = ts; row < a.rows; row += kReduceSlices) {
      const Pack<float, VEC> v = load_pack<float, VEC>(p + row * a.N);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] += v.get(e);
    }
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
    store_f32<VEC>(a.dgamma + col, o);
  }
}

// ---------------------------------------------------------------------------
// Host-side dispatch to the compiled instantiations.
// ---------------------------------------------------------------------------
template <typename S, int VEC, int ITERS>
hipError_t fwd_inst(const RowPlan& p, const FwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((rmsnorm_fwd_kernel<S, VEC, ITERS>), dim3(static_cast<unsigned>(p.grid)), dim3(p.threads()), 0, s,
                     a);
  return hipGetLastError();
}

template <typename S, int VEC, int ITERS>
hipError_t bwd_inst(const RowPlan& p, const BwdArgs& a, hipStream_t s) {
  const size_t lds = static_cast<size_t>(a.N) * sizeof(float);
  hipLaunchKernelGGL((rmsnorm_bwd_rows_kernel<S, VEC, ITERS>), dim3(static_cast<unsigned>(p.grid)),
                     dim3(p.threads()), lds, s, a);
  return hipGetLastError();
}

template <typename S, int VEC, typename Args, hipError_t (*L1)(const RowPlan&, const Args&, hipStream_t),
          hipError_t (*L2)(const RowPlan&, const Args&, hipStream_t), hipError_t (*L4)(const RowPlan&, const Args&, hipStream_t),
          hipError_t (*L5)(const RowPlan&, const Args&, hipStream_t), hipError_t (*L8)(const RowPlan&, const Args&, hipStream_t),
          hipError_t (*L16)(const RowPlan&, const Args&, hipStream_t)>
hipError_t pick_iters(const RowPlan& p, const Args& a, hipStream_t s) {
  switch (p.iters) {
    case 1: return L1(p, a, s);
    case 2: return L2(p, a, s);
    case 4: return L4(p, a, s);
    case 5: return L5(p, a, s);
    case 8: return L8(p, a, s);
    case 16: return L16(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename S, int VEC>
hipError_t fwd_vec(const RowPlan& p, const FwdArgs& a, hipStream_t s) {
  return pick_iters<S, VEC, FwdArgs, fwd_inst<S, VEC, 1>, fwd_inst<S, VEC, 2>, fwd_inst<S, VEC, 4>, fwd_inst<S, VEC, 5>,
                    fwd_inst<S, VEC, 8>, fwd_inst<S, VEC, 16>>(p, a, s);
}

template <typename S, int VEC>
hipError_t bwd_vec(const RowPlan& p, const BwdArgs& a, hipStream_t s) {
  return pick_iters<S, VEC, BwdArgs, bwd_inst<S, VEC, 1>, bwd_inst<S, VEC, 2>, bwd_inst<S, VEC, 4>, bwd_inst<S, VEC, 5>,
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
  } else {
    switch (p.vec) {
      case 1: return fwd_vec<uint16_t, 1>(p, a, s);
      case 2: return fwd_vec<uint16_t, 2>(p, a, s);
      case 4: return fwd_vec<uint16_t, 4>(p, a, s);
      case 8: return fwd_vec<uint16_t, 8>(p, a, s);
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
  } else {
    switch (p.vec) {
      case 1: return bwd_vec<uint16_t, 1>(p, a, s);
      case 2: return bwd_vec<uint16_t, 2>(p, a, s);
      case 4: return bwd_vec<uint16_t, 4>(p, a, s);
      case 8: return bwd_vec<uint16_t, 8>(p, a, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_dgamma_reduce(int vec, const ReduceArgs& a, hipStream_t s) {
  const int cols = kReduceCols * vec;
  const unsigned grid = static_cast<unsigned>((a.N + cols - 1) / cols);
  if (vec == 4) {
    hipLaunchKernelGGL(rmsnorm_dgamma_reduce_kernel<4>, dim3(grid), dim3(kReduceCols * kReduceSlices), 0, s, a);
  } else if (vec == 1) {
    hipLaunchKernelGGL(rmsnorm_dgamma_reduce_kernel<1>, dim3(grid), dim3(kReduceCols * kReduceSlices), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rmsn
