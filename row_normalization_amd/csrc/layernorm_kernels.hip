// gfx950 (CDNA4) kernels for fused LayerNorm forward and backward.
//
// What is computed (the LayerNorm chapter "第 07 章:LayerNorm——反向传播与原子锁"
// of a Triton tutorial series, chuoer47.github.io; section 1 for the forward,
// sections 3.0 and 3.3 for the input gradient, 3.3-3.5 for the weight and
// bias gradients):
//   forward   mean = sum(x)/N, var = sum((x - mean)^2)/N, rstd = 1/sqrt(var + eps),
//             y = (x - mean) * rstd * w + b
//   backward  x_hat = (x - mean) * rstd, g = w * dy, c1 = sum(x_hat * g)/N,
//             c2 = sum(g)/N, dx = (g - (x_hat * c1 + c2)) * rstd,
//             dw = sum_rows dy * x_hat, db = sum_rows dy
//
// The kernels share the RMSNorm kernels' skeleton (device_common.h): whole
// 16-byte column vectors per lane, every row access an unconditional raw
// buffer operation through a per-row descriptor (the hardware range check
// masks the tail and the rows past M), nontemporal streaming of x, dy, y and
// dx, DPP wave sums and one LDS barrier per cross-wave sum.
//  - The forward keeps the row in registers and takes the page's two passes
//    over it there: the mean first, then the sum of squared differences from
//    it (no E[x^2] - mean^2 cancellation), so x is read from HBM once.  The
//    second pass masks the vectors past N, whose zeros would otherwise add
//    mean^2 each.
//  - The backward needs two row sums, c1 and c2; they travel together through
//    one barrier.  Past-the-end vectors need no mask there: their dy and w
//    read as zero, so they add nothing to either sum or to the gradients.
//  - Instead of the page's lock-protected accumulation into GROUP_SIZE
//    intermediate rows, the backward is a persistent grid: each workgroup
//    keeps its dw and db column partials in fp32 registers across its rows
//    and writes one partial row of each; the RMSNorm column-sum kernel then
//    adds the partial rows in a fixed order (both tables in one launch).  No
//    locks, no atomics: every result is bitwise reproducible.
//  - dx may be written over dy (each lane loads its dy elements before it
//    stores the same elements of dx).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "launch.h"

namespace rmsn {
namespace {
using namespace dev;

// Streamed operands are touched once per pass: nontemporal, as for RMSNorm.
constexpr int kLnLoadX = kNontemporal;
constexpr int kLnStoreY = kNontemporal;
constexpr int kLnLoadXdy = kNontemporal;
constexpr int kLnStoreDx = kNontemporal;

// ---------------------------------------------------------------------------
// Forward.  Grid as for the RMSNorm forward (row groups, or persistent where
// that fills the CUs evenly); weight and bias are loaded once per workgroup.
// ---------------------------------------------------------------------------
template <typename S, int VEC, int ITERS>
__global__ __launch_bounds__(1024) void layernorm_fwd_kernel(const LnFwdArgs a) {
  constexpr uint32_t kPack = Pack<S, VEC>::kBytes;
  const Lane L(a.wpr);
  __shared__ float red[2][kMaxBlockWaves];

  const uint32_t voff = L.first_vec() * kPack;
  const uint32_t iter_bytes = static_cast<uint32_t>(a.wpr) * kWave * kPack;
  const uint32_t row_bytes = static_cast<uint32_t>(a.N) * sizeof(S);
  const Rsrc rw = make_rsrc(a.weight, row_bytes);
  const Rsrc rb = make_rsrc(a.bias, row_bytes);
  const Rsrc rmean = make_rsrc(a.mean, static_cast<uint32_t>(a.M) * 4u);
  const Rsrc rrstd = make_rsrc(a.rstd, static_cast<uint32_t>(a.M) * 4u);
  const S* x = static_cast<const S*>(a.x);
  S* y = static_cast<S*>(a.y);

  // weight and bias once per workgroup, kept packed across its rows
  Pack<S, VEC> wv[ITERS];
  Pack<S, VEC> bv[ITERS];
#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    wv[i] = buf_load<S, VEC, kDefault>(rw, voff + i * iter_bytes);
    bv[i] = buf_load<S, VEC, kDefault>(rb, voff + i * iter_bytes);
  }

  for (int64_t step = 0; step < a.row_iters; ++step) {
    const int64_t row = row_of(step, a.row_iters, a.rpb, L.group);
    const bool active = row < a.M;
    const int64_t off = active ? row * a.stride : 0;
    const Rsrc rx = make_rsrc(x + off, active ? row_bytes : 0u);
    const Rsrc ry = make_rsrc(y + off, active ? row_bytes : 0u);

    Pack<S, VEC> xv[ITERS];
#pragma unroll
    for (int i = 0; i < ITERS; ++i) xv[i] = buf_load<S, VEC, kLnLoadX>(rx, voff + i * iter_bytes);
    // weight and bias are unpacked inside the loop, after the row's loads
    // are issued: unpacked before it, the first row's x loads wait for them
    // (measured 7-14 % slower at 4096 x 10240 and 4096 x 12288 fp16).  The
    // RMSNorm forward, with one operand less, keeps its weight unpacked
    // across the rows and issues the first row's loads ahead of that instead.
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      wv[i].keep_packed();
      bv[i].keep_packed();
    }

    // pass 1: the mean (vectors past N read as zero and add nothing)
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < ITERS; ++i)
#pragma unroll
      for (int e = 0; e < VEC; ++e) s += xv[i].get(e);
#pragma unroll
    for (int i = 0; i < ITERS; ++i) xv[i].keep_packed();
    s = wave_sum(s);
    if (a.wpr > 1) s = group_sum(s, red, 2 * step, L.wave, L.group, a.wpr, L.lane);
    const float mean = s * a.inv_n;

    // pass 2: squared differences from the mean, over the columns < N only
    float d = 0.f;
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const bool in_row = static_cast<int>((i * a.wpr + L.wv) * kWave + L.lane) < a.nvec;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float t = in_row ? xv[i].get(e) - mean : 0.f;
        d = fmaf(t, t, d);
      }
    }
#pragma unroll
    for (int i = 0; i < ITERS; ++i) xv[i].keep_packed();
    d = wave_sum(d);
    if (a.wpr > 1) d = group_sum(d, red, 2 * step + 1, L.wave, L.group, a.wpr, L.lane);
    const float rstd = rsqrtf(fmaf(d, a.inv_n, a.eps));

    // one lane per row writes mean and rstd; the others' offsets are out of range
    const bool writer = active && L.wv == 0 && L.lane == 0;
    const uint32_t soff = writer ? static_cast<uint32_t>(row) * 4u : kOutOfRange;
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, mean), rmean, soff, 0, kDefault);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, rstd), rrstd, soff, 0, kDefault);

#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      float o[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[e] = fmaf((xv[i].get(e) - mean) * rstd, wv[i].get(e), bv[i].get(e));
      buf_store<S, VEC, kLnStoreY>(round_pack<S, VEC>(o), ry, voff + i * iter_bytes);
    }
  }
}

// ---------------------------------------------------------------------------
// Backward row pass: dx, and per-workgroup partial rows of dw and db.
// Persistent: workgroup b takes rows (k * grid + b) * rpb + group.  A lane
// keeps, for the columns it owns, w in fp32 and its dw and db partials in
// fp32 registers across all of its rows.
// ---------------------------------------------------------------------------
// One row's operands as a lane holds them between its loads and its work.
template <typename S, int VEC, int ITERS>
struct LnBwdRow {
  Pack<S, VEC> x[ITERS];
  Pack<S, VEC> dy[ITERS];
  float mean;
  float rstd;
};

// Offsets and descriptors a backward lane uses for every row.
struct LnBwdGeom {
  uint32_t voff;        // byte offset of the lane's first vector in a row
  uint32_t iter_bytes;  // bytes between the lane's successive vectors
  uint32_t row_bytes;   // N * sizeof(S)
  Rsrc mean;            // the M saved means
  Rsrc rstd;            // the M saved rstd values
};

template <typename S, int VEC, int ITERS>
__device__ __forceinline__ void ln_bwd_load_row(LnBwdRow<S, VEC, ITERS>& t, const LnBwdArgs& a, int64_t step,
                                                const Lane& L, const LnBwdGeom& G) {
  const int64_t row = row_of(step, a.row_iters, a.rpb, L.group);
  const bool active = row < a.M;
  const int64_t off = active ? row * a.stride : 0;
  const Rsrc rx = make_rsrc(static_cast<const S*>(a.x) + off, active ? G.row_bytes : 0u);
  const Rsrc rd = make_rsrc(static_cast<const S*>(a.dy) + off, active ? G.row_bytes : 0u);
#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    t.x[i] = buf_load<S, VEC, kLnLoadXdy>(rx, G.voff + i * G.iter_bytes);
    t.dy[i] = buf_load<S, VEC, kLnLoadXdy>(rd, G.voff + i * G.iter_bytes);
  }
  // mean and rstd of a missing row read as zero (out of the descriptors' range)
  const uint32_t soff = active ? static_cast<uint32_t>(row) * 4u : kOutOfRange;
  t.mean = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(G.mean, soff, 0, kDefault));
  t.rstd = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(G.rstd, soff, 0, kDefault));
}

template <typename S, int VEC, int ITERS>
__device__ __forceinline__ void ln_bwd_process_row(LnBwdRow<S, VEC, ITERS>& t, const LnBwdArgs& a, int64_t step,
                                                   const float (&w)[ITERS][VEC], float (&accw)[ITERS][VEC],
                                                   float (&accb)[ITERS][VEC], float (*red)[2][kMaxBlockWaves],
                                                   const Lane& L, const LnBwdGeom& G) {
  const int64_t row = row_of(step, a.row_iters, a.rpb, L.group);
  const bool active = row < a.M;
  const int64_t off = active ? row * a.stride : 0;
  // dx may be the dy buffer itself; every element of dy this lane owns was
  // loaded into registers before this point
  const Rsrc rdx = make_rsrc(static_cast<S*>(a.dx) + off, active ? G.row_bytes : 0u);
  const float mean = t.mean, rstd = t.rstd;

  // the two row sums: of x_hat * g and of g, with g = w * dy
  float s1 = 0.f, s2 = 0.f;
#pragma unroll
  for (int i = 0; i < ITERS; ++i)
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const float xh = (t.x[i].get(e) - mean) * rstd;
      const float g = w[i][e] * t.dy[i].get(e);
      s1 = fmaf(xh, g, s1);
      s2 += g;
    }
#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    t.x[i].keep_packed();
    t.dy[i].keep_packed();
  }
  s1 = wave_sum(s1);
  s2 = wave_sum(s2);
  if (a.wpr > 1) group_sum2(s1, s2, red, step, L.wave, L.group, a.wpr, L.lane);
  const float c1 = s1 * a.inv_n;
  const float c2 = s2 * a.inv_n;

#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    float o[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const float df = t.dy[i].get(e);
      const float xh = (t.x[i].get(e) - mean) * rstd;
      o[e] = (w[i][e] * df - fmaf(xh, c1, c2)) * rstd;
      accw[i][e] = fmaf(df, xh, accw[i][e]);
      accb[i][e] += df;
    }
    buf_store<S, VEC, kLnStoreDx>(round_pack<S, VEC>(o), rdx, G.voff + i * G.iter_bytes);
  }
}

template <typename S, int VEC, int ITERS, int MAXT>
__global__ __launch_bounds__(MAXT) void layernorm_bwd_rows_kernel(const LnBwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) float comb[];  // 2N floats, when rpb > 1
  __shared__ float red[2][2][kMaxBlockWaves];
  constexpr uint32_t kPack = Pack<S, VEC>::kBytes;
  const Lane L(a.wpr);
  LnBwdGeom G;
  G.voff = L.first_vec() * kPack;
  G.iter_bytes = static_cast<uint32_t>(a.wpr) * kWave * kPack;
  G.row_bytes = static_cast<uint32_t>(a.N) * sizeof(S);
  G.mean = make_rsrc(a.mean, static_cast<uint32_t>(a.M) * 4u);
  G.rstd = make_rsrc(a.rstd, static_cast<uint32_t>(a.M) * 4u);
  const uint32_t voff = G.voff;

  float w[ITERS][VEC];
  float accw[ITERS][VEC];
  float accb[ITERS][VEC];
  {
    const Rsrc rw = make_rsrc(a.weight, G.row_bytes);
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const Pack<S, VEC> g = buf_load<S, VEC, kDefault>(rw, voff + i * G.iter_bytes);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        w[i][e] = g.get(e);
        accw[i][e] = 0.f;
        accb[i][e] = 0.f;
      }
    }
  }

  bool pipelined = false;
  if constexpr (bwd_pipeline_fits(RowOp::kLnBwd, dtype_code<S>(), VEC, ITERS, MAXT)) pipelined = a.pipeline;
  if (pipelined) {
    // One workgroup per CU: the next row's loads are in flight during this
    // row's sums, barrier and stores.  Unconditional loads over an even
    // number of steps and scheduling barriers between the rows, for the
    // reasons given in the RMSNorm backward (rows past M load zeros, store
    // nothing and add nothing to the partials).
    LnBwdRow<S, VEC, ITERS> ta, tb;
    ln_bwd_load_row(ta, a, 0, L, G);
    __builtin_amdgcn_sched_barrier(0);
    for (int64_t step = 0; step < a.row_iters; step += 2) {
      ln_bwd_load_row(tb, a, step + 1, L, G);
      __builtin_amdgcn_sched_barrier(0);
      ln_bwd_process_row(ta, a, step, w, accw, accb, red, L, G);
      ln_bwd_load_row(ta, a, step + 2, L, G);
      __builtin_amdgcn_sched_barrier(0);
      ln_bwd_process_row(tb, a, step + 1, w, accw, accb, red, L, G);
    }
  } else {
    // One row at a time.  This loop carries the same row work as
    // ln_bwd_load_row + ln_bwd_process_row, written out in place: split into
    // the two helpers it needs ~10 more registers and spills in the widest
    // fp32 fallback instantiation (1-element vectors, 16 per lane).
    for (int64_t step = 0; step < a.row_iters; ++step) {
      const int64_t row = row_of(step, a.row_iters, a.rpb, L.group);
      const bool active = row < a.M;
      const int64_t off = active ? row * a.stride : 0;
      const Rsrc rx = make_rsrc(static_cast<const S*>(a.x) + off, active ? G.row_bytes : 0u);
      const Rsrc rd = make_rsrc(static_cast<const S*>(a.dy) + off, active ? G.row_bytes : 0u);
      const Rsrc rdx = make_rsrc(static_cast<S*>(a.dx) + off, active ? G.row_bytes : 0u);

      Pack<S, VEC> xv[ITERS];
      Pack<S, VEC> dv[ITERS];
#pragma unroll
      for (int i = 0; i < ITERS; ++i) {
        xv[i] = buf_load<S, VEC, kLnLoadXdy>(rx, voff + i * G.iter_bytes);
        dv[i] = buf_load<S, VEC, kLnLoadXdy>(rd, voff + i * G.iter_bytes);
      }
      // mean and rstd of a missing row read as zero (out of the descriptors' range)
      const uint32_t soff = active ? static_cast<uint32_t>(row) * 4u : kOutOfRange;
      const float mean = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(G.mean, soff, 0, kDefault));
      const float rstd = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(G.rstd, soff, 0, kDefault));

      // the two row sums: of x_hat * g and of g, with g = w * dy
      float s1 = 0.f, s2 = 0.f;
#pragma unroll
      for (int i = 0; i < ITERS; ++i)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float xh = (xv[i].get(e) - mean) * rstd;
          const float g = w[i][e] * dv[i].get(e);
          s1 = fmaf(xh, g, s1);
          s2 += g;
        }
#pragma unroll
      for (int i = 0; i < ITERS; ++i) {
        xv[i].keep_packed();
        dv[i].keep_packed();
      }
      s1 = wave_sum(s1);
      s2 = wave_sum(s2);
      if (a.wpr > 1) group_sum2(s1, s2, red, step, L.wave, L.group, a.wpr, L.lane);
      const float c1 = s1 * a.inv_n;
      const float c2 = s2 * a.inv_n;

#pragma unroll
      for (int i = 0; i < ITERS; ++i) {
        float o[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float df = dv[i].get(e);
          const float xh = (xv[i].get(e) - mean) * rstd;
          o[e] = (w[i][e] * df - fmaf(xh, c1, c2)) * rstd;
          accw[i][e] = fmaf(df, xh, accw[i][e]);
          accb[i][e] += df;
        }
        buf_store<S, VEC, kLnStoreDx>(round_pack<S, VEC>(o), rdx, voff + i * G.iter_bytes);
      }
    }
  }

  // One dw and one db partial row per workgroup; row groups are added in LDS
  // in group order, and the last group adds that sum to its own and writes
  // the two partial rows (every group covers every column; lanes past the
  // row's end store out of the descriptors' range).
  float* pw = a.partials + static_cast<int64_t>(blockIdx.x) * a.N;
  float* pb = a.partials + (static_cast<int64_t>(gridDim.x) + blockIdx.x) * a.N;
  for (int g = 0; g < a.rpb - 1; ++g) {
    if (g > 0) __syncthreads();
    if (L.group == g) {
#pragma unroll
      for (int i = 0; i < ITERS; ++i) {
        const int v = (i * a.wpr + L.wv) * kWave + L.lane;
        if (v < a.nvec) {
          if (g == 0) {
            comb_store<VEC>(comb, v, a.nvec, accw[i]);
            comb_store<VEC>(comb + a.N, v, a.nvec, accb[i]);
          } else {
            // Both tables' cells are read before either is written (measured:
            // 4096 x 1024 fp16, 8 row groups per workgroup, 15.9 -> 10.5 us
            // against interleaved read-add-write steps).
            float tw[VEC], tb[VEC];
            comb_load<VEC>(comb, v, a.nvec, tw);
            comb_load<VEC>(comb + a.N, v, a.nvec, tb);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
              tw[e] += accw[i][e];
              tb[e] += accb[i][e];
            }
            comb_store<VEC>(comb, v, a.nvec, tw);
            comb_store<VEC>(comb + a.N, v, a.nvec, tb);
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
      const int v = (i * a.wpr + L.wv) * kWave + L.lane;
      if (v < a.nvec) {
        float tw[VEC], tb[VEC];
        comb_load<VEC>(comb, v, a.nvec, tw);
        comb_load<VEC>(comb + a.N, v, a.nvec, tb);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          accw[i][e] += tw[e];
          accb[i][e] += tb[e];
        }
      }
    }
  }
  const Rsrc rdw = make_rsrc(pw, static_cast<uint32_t>(a.N) * 4u);
  const Rsrc rdb = make_rsrc(pb, static_cast<uint32_t>(a.N) * 4u);
  const uint32_t voff32 = L.first_vec() * VEC * 4u;
  const uint32_t iter32 = static_cast<uint32_t>(a.wpr) * kWave * VEC * 4u;
  if (a.partials_nt) {
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      buf_store_f32<VEC, kNontemporal>(accw[i], rdw, voff32 + i * iter32);
      buf_store_f32<VEC, kNontemporal>(accb[i], rdb, voff32 + i * iter32);
    }
  } else {
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      buf_store_f32<VEC, kDefault>(accw[i], rdw, voff32 + i * iter32);
      buf_store_f32<VEC, kDefault>(accb[i], rdb, voff32 + i * iter32);
    }
  }
}

// ---------------------------------------------------------------------------
// Wide rows: 16-bit rows beyond the register plans (up to kLnWideMaxN
// elements, the 64 KB per row of the chapter's Step 2 wrapper), one 1024-thread
// workgroup per row.  Lane t owns vector k * 1024 + t of the row for each
// chunk k < chunks (at most kLnWideColsPerLane columns per lane); vectors at
// or past N / VEC read zero and store nothing through the row descriptors.
// ---------------------------------------------------------------------------
constexpr int kWideThreads = 1024;

// Sums of one value per lane over the workgroup's 16 waves (as group_sum2,
// slots alternating with the step parity).
__device__ __forceinline__ void block_sum2(float& s1, float& s2, float (*red)[2][kMaxBlockWaves], int64_t step,
                                           const Lane& L) {
  s1 = wave_sum(s1);
  s2 = wave_sum(s2);
  group_sum2(s1, s2, red, step, L.wave, 0, kWideThreads / kWave, L.lane);
}

// Forward over a row held in registers (x loaded once per row); weight and
// bias are read per row from the caches (N elements shared by every row).
template <typename S, int VEC>
__global__ __launch_bounds__(kWideThreads) void layernorm_fwd_wide_kernel(const LnFwdArgs a) {
  constexpr int KMAX = kLnWideColsPerLane / VEC;
  constexpr uint32_t kPack = Pack<S, VEC>::kBytes;
  const Lane L(kWideThreads / kWave);
  __shared__ float red[2][2][kMaxBlockWaves];
  const int chunks = a.chunks;
  const int64_t steps = a.row_iters;
  const uint32_t voff = threadIdx.x * kPack;
  constexpr uint32_t kChunkBytes = kWideThreads * kPack;
  const uint32_t row_bytes = static_cast<uint32_t>(a.N) * sizeof(S);
  const Rsrc rw = make_rsrc(a.weight, row_bytes);
  const Rsrc rb = make_rsrc(a.bias, row_bytes);
  const Rsrc rmean = make_rsrc(a.mean, static_cast<uint32_t>(a.M) * 4u);
  const Rsrc rrstd = make_rsrc(a.rstd, static_cast<uint32_t>(a.M) * 4u);
  for (int64_t step = 0; step < steps; ++step) {
    const int64_t row = step * gridDim.x + blockIdx.x;
    const bool active = row < a.M;
    const int64_t off = active ? row * a.stride : 0;
    const Rsrc rx = make_rsrc(static_cast<const S*>(a.x) + off, active ? row_bytes : 0u);
    const Rsrc ry = make_rsrc(static_cast<S*>(a.y) + off, active ? row_bytes : 0u);
    Pack<S, VEC> xv[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
      xv[k] = buf_load<S, VEC, kLnLoadX>(rx, k < chunks ? voff + k * kChunkBytes : kOutOfRange);
    float s = 0.f, unused = 0.f;
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
#pragma unroll
      for (int e = 0; e < VEC; ++e) s += xv[k].get(e);
    block_sum2(s, unused, red, 2 * step, L);
    const float mean = s * a.inv_n;
    float d = 0.f;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      const bool in_row = static_cast<int>(k * kWideThreads + threadIdx.x) < a.nvec;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float t = in_row ? xv[k].get(e) - mean : 0.f;
        d = fmaf(t, t, d);
      }
    }
    block_sum2(d, unused, red, 2 * step + 1, L);
    const float rstd = rsqrtf(fmaf(d, a.inv_n, a.eps));
    const uint32_t soff = active && threadIdx.x == 0 ? static_cast<uint32_t>(row) * 4u : kOutOfRange;
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, mean), rmean, soff, 0, kDefault);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, rstd), rrstd, soff, 0, kDefault);
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      const uint32_t o = k < chunks ? voff + k * kChunkBytes : kOutOfRange;
      const Pack<S, VEC> wv = buf_load<S, VEC, kDefault>(rw, o);
      const Pack<S, VEC> bv = buf_load<S, VEC, kDefault>(rb, o);
      float out[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) out[e] = fmaf((xv[k].get(e) - mean) * rstd, wv.get(e), bv.get(e));
      buf_store<S, VEC, kLnStoreY>(round_pack<S, VEC>(out), ry, o);
    }
  }
}

// A value every lane of the workgroup holds alike, moved to a scalar register.
__device__ __forceinline__ float uniform_f32(uint32_t bits) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(bits));
}

// Backward over rows read in 16-byte vectors: per row, the two row sums
// (pass 1), then dx and the dw / db contributions (pass 2), with the
// workgroup's next row on its way during pass 2.  Rows of CH chunks (3 or 4:
// 16385-32768 elements).  x and dy of a row stay in registers between the
// passes; dw and db partials stay in fp32 registers across the workgroup's
// rows (one partial row of each at the end).  The weight is copied into LDS
// once per workgroup (CH * 16 KB; gfx950 gives a workgroup up to 160 KB) and
// read from there, so no load of pass 2 queues behind the next row's loads,
// which the vector-memory counter retires in issue order.  As soon as pass 2
// has used chunk k of the row (dx stored, dw and db added), it loads chunk k
// of the next row into the same registers: one register set, which is what
// fits a lane of a 1024-thread workgroup (128 registers; two full sets would
// not).  Offsets at or past a row's bytes -- the unfilled end of the last
// chunk, and every offset once the workgroup has no next row -- read zero
// and store nothing through the row descriptors.
template <typename S, int CH>
__global__ __launch_bounds__(kWideThreads) void layernorm_bwd_wide_held_kernel(const LnBwdArgs a) {
  constexpr int VEC = 16 / static_cast<int>(sizeof(S));
  typedef Pack<S, VEC> P;
  const Lane L(kWideThreads / kWave);
  __shared__ float red[2][2][kMaxBlockWaves];
  extern __shared__ u32x4_t wlds[];  // CH * kWideThreads weight vectors, zero past the row
  const int64_t steps = a.row_iters;
  const uint32_t t = threadIdx.x;
  const uint32_t voff = t * 16u;
  constexpr uint32_t kChunkBytes = kWideThreads * 16u;
  const uint32_t row_bytes = static_cast<uint32_t>(a.N) * sizeof(S);
  const Rsrc rw = make_rsrc(a.weight, row_bytes);
  const Rsrc rmean = make_rsrc(a.mean, static_cast<uint32_t>(a.M) * 4u);
  const Rsrc rrstd = make_rsrc(a.rstd, static_cast<uint32_t>(a.M) * 4u);
#pragma unroll
  for (int k = 0; k < CH; ++k)
    wlds[k * kWideThreads + t] = __builtin_amdgcn_raw_buffer_load_b128(rw, voff + k * kChunkBytes, 0, kDefault);
  float accw[CH][VEC], accb[CH][VEC];
#pragma unroll
  for (int k = 0; k < CH; ++k)
#pragma unroll
    for (int e = 0; e < VEC; ++e) accw[k][e] = accb[k][e] = 0.f;

  // the first row (grid <= M, so every workgroup has one)
  int64_t row = blockIdx.x;
  bool active = row < a.M;
  Rsrc rx = make_rsrc(static_cast<const S*>(a.x) + (active ? row * a.stride : 0), active ? row_bytes : 0u);
  Rsrc rd = make_rsrc(static_cast<const S*>(a.dy) + (active ? row * a.stride : 0), active ? row_bytes : 0u);
  const uint32_t soff = active ? static_cast<uint32_t>(row) * 4u : kOutOfRange;
  float mean = uniform_f32(__builtin_amdgcn_raw_buffer_load_b32(rmean, soff, 0, kDefault));
  float rstd = uniform_f32(__builtin_amdgcn_raw_buffer_load_b32(rrstd, soff, 0, kDefault));
  P xv[CH], dv[CH];
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    xv[k] = buf_load<S, VEC, kLnLoadXdy>(rx, voff + k * kChunkBytes);
    dv[k] = buf_load<S, VEC, kLnLoadXdy>(rd, voff + k * kChunkBytes);
  }
  __syncthreads();  // the weight is in LDS
  // Only the last chunk can lie wholly past the row for a wave (at N = 16392
  // it holds one vector, so 15 of the 16 waves have none there).  Such a wave
  // skips that chunk: its zeros would change no bit of the sums (which start
  // at +0) or of the partials, and its loads and stores touch no memory.
  // Rows of three chunks only: in the four-chunk instantiation the branch
  // needs registers it does not have (it spilled).  Measured on MI355X
  // (interleaved, full backward, bit-identical results): fp16 4096 x 16392
  // 4.3 %, 4096 x 18432 3.8 %, 16384 x 16392 3.3 %, 4096 x 20480 2.6 %
  // faster; full last chunks unchanged.
  const bool last_live = CH != 3 || static_cast<int>((CH - 1) * kWideThreads + L.wave * kWave) < a.nvec;

  for (int64_t step = 0; step < steps; ++step) {
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      if (CH == 3 && k == CH - 1 && !last_live) continue;
      const P w = __builtin_bit_cast(P, wlds[k * kWideThreads + t]);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float xh = (xv[k].get(e) - mean) * rstd;
        const float g = w.get(e) * dv[k].get(e);
        s1 = fmaf(xh, g, s1);
        s2 += g;
      }
    }
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      xv[k].keep_packed();
      dv[k].keep_packed();
    }
    block_sum2(s1, s2, red, step, L);
    const float c1 = uniform_f32(__builtin_bit_cast(uint32_t, s1 * a.inv_n));
    const float c2 = uniform_f32(__builtin_bit_cast(uint32_t, s2 * a.inv_n));

    const Rsrc rdx = make_rsrc(static_cast<S*>(a.dx) + (active ? row * a.stride : 0), active ? row_bytes : 0u);
    const int64_t nrow = row + gridDim.x;
    const bool nactive = step + 1 < steps && nrow < a.M;
    const Rsrc nrx = make_rsrc(static_cast<const S*>(a.x) + (nactive ? nrow * a.stride : 0), nactive ? row_bytes : 0u);
    const Rsrc nrd = make_rsrc(static_cast<const S*>(a.dy) + (nactive ? nrow * a.stride : 0), nactive ? row_bytes : 0u);
    const uint32_t nsoff = nactive ? static_cast<uint32_t>(nrow) * 4u : kOutOfRange;
    const float nmean = uniform_f32(__builtin_amdgcn_raw_buffer_load_b32(rmean, nsoff, 0, kDefault));
    const float nrstd = uniform_f32(__builtin_amdgcn_raw_buffer_load_b32(rrstd, nsoff, 0, kDefault));
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      if (CH == 3 && k == CH - 1 && !last_live) continue;
      const uint32_t o = voff + k * kChunkBytes;
      const P w = __builtin_bit_cast(P, wlds[k * kWideThreads + t]);
      float out[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float df = dv[k].get(e);
        const float xh = (xv[k].get(e) - mean) * rstd;
        out[e] = (w.get(e) * df - fmaf(xh, c1, c2)) * rstd;
        accw[k][e] = fmaf(df, xh, accw[k][e]);
        accb[k][e] += df;
      }
      buf_store<S, VEC, kLnStoreDx>(round_pack<S, VEC>(out), rdx, o);
      // chunk k's arithmetic stays ahead of the loads that reuse its
      // registers (else the scheduler defers the dw sums and spills)
      __builtin_amdgcn_sched_barrier(0);
      // rows never overlap, so the next row's dy is not this row's dx
      xv[k] = buf_load<S, VEC, kLnLoadXdy>(nrx, o);
      dv[k] = buf_load<S, VEC, kLnLoadXdy>(nrd, o);
    }
    row = nrow;
    active = nactive;
    mean = nmean;
    rstd = nrstd;
  }
  const Rsrc rpw = make_rsrc(a.partials + static_cast<int64_t>(blockIdx.x) * a.N, static_cast<uint32_t>(a.N) * 4u);
  const Rsrc rpb =
      make_rsrc(a.partials + (static_cast<int64_t>(gridDim.x) + blockIdx.x) * a.N, static_cast<uint32_t>(a.N) * 4u);
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const uint32_t o = (k * kWideThreads + t) * VEC * 4u;
    if (a.partials_nt) {
      buf_store_f32<VEC, kNontemporal>(accw[k], rpw, o);
      buf_store_f32<VEC, kNontemporal>(accb[k], rpb, o);
    } else {
      buf_store_f32<VEC, kDefault>(accw[k], rpw, o);
      buf_store_f32<VEC, kDefault>(accb[k], rpb, o);
    }
  }
}

// Backward over rows read in narrower vectors (N not a multiple of 8, or
// misaligned rows): a row in such vectors would need more registers than a
// lane of a 1024-thread workgroup has, so pass 2 reads x and dy again, from
// L2 (pass 1 loads them with the allocating policy), and the weight is read
// per pass from the caches.  One row at a time; dw and db partials as above.
template <typename S, int VEC>
__global__ __launch_bounds__(kWideThreads) void layernorm_bwd_wide_kernel(const LnBwdArgs a) {
  constexpr int KMAX = kLnWideColsPerLane / VEC;
  constexpr uint32_t kPack = Pack<S, VEC>::kBytes;
  static_assert(kPack < 16, "16-byte vectors take the held-row kernel");
  const Lane L(kWideThreads / kWave);
  __shared__ float red[2][2][kMaxBlockWaves];
  const int chunks = a.chunks;
  const int64_t steps = a.row_iters;
  const uint32_t voff = threadIdx.x * kPack;
  constexpr uint32_t kChunkBytes = kWideThreads * kPack;
  const uint32_t row_bytes = static_cast<uint32_t>(a.N) * sizeof(S);
  const Rsrc rw = make_rsrc(a.weight, row_bytes);
  const Rsrc rmean = make_rsrc(a.mean, static_cast<uint32_t>(a.M) * 4u);
  const Rsrc rrstd = make_rsrc(a.rstd, static_cast<uint32_t>(a.M) * 4u);
  float accw[KMAX][VEC], accb[KMAX][VEC];
#pragma unroll
  for (int k = 0; k < KMAX; ++k)
#pragma unroll
    for (int e = 0; e < VEC; ++e) accw[k][e] = accb[k][e] = 0.f;

  for (int64_t step = 0; step < steps; ++step) {
    const int64_t row = step * gridDim.x + blockIdx.x;
    const bool active = row < a.M;
    const int64_t off = active ? row * a.stride : 0;
    const Rsrc rx = make_rsrc(static_cast<const S*>(a.x) + off, active ? row_bytes : 0u);
    const Rsrc rd = make_rsrc(static_cast<const S*>(a.dy) + off, active ? row_bytes : 0u);
    const Rsrc rdx = make_rsrc(static_cast<S*>(a.dx) + off, active ? row_bytes : 0u);
    const uint32_t soff = active ? static_cast<uint32_t>(row) * 4u : kOutOfRange;
    const float mean = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rmean, soff, 0, kDefault));
    const float rstd = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rrstd, soff, 0, kDefault));

    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      const uint32_t o = k < chunks ? voff + k * kChunkBytes : kOutOfRange;
      const Pack<S, VEC> x = buf_load<S, VEC, kDefault>(rx, o);
      const Pack<S, VEC> dy = buf_load<S, VEC, kDefault>(rd, o);
      const Pack<S, VEC> w = buf_load<S, VEC, kDefault>(rw, o);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float xh = (x.get(e) - mean) * rstd;
        const float g = w.get(e) * dy.get(e);
        s1 = fmaf(xh, g, s1);
        s2 += g;
      }
    }
    block_sum2(s1, s2, red, step, L);
    const float c1 = s1 * a.inv_n;
    const float c2 = s2 * a.inv_n;

#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      const uint32_t o = k < chunks ? voff + k * kChunkBytes : kOutOfRange;
      // every element of dy this lane reads here it has not yet overwritten
      // (dx may be dy itself: this lane stores only the elements it loads)
      const Pack<S, VEC> x = buf_load<S, VEC, kLnLoadXdy>(rx, o);
      const Pack<S, VEC> dy = buf_load<S, VEC, kLnLoadXdy>(rd, o);
      const Pack<S, VEC> w = buf_load<S, VEC, kDefault>(rw, o);
      float out[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float df = dy.get(e);
        const float xh = (x.get(e) - mean) * rstd;
        out[e] = (w.get(e) * df - fmaf(xh, c1, c2)) * rstd;
        accw[k][e] = fmaf(df, xh, accw[k][e]);
        accb[k][e] += df;
      }
      buf_store<S, VEC, kLnStoreDx>(round_pack<S, VEC>(out), rdx, o);
    }
  }
  const Rsrc rpw = make_rsrc(a.partials + static_cast<int64_t>(blockIdx.x) * a.N, static_cast<uint32_t>(a.N) * 4u);
  const Rsrc rpb =
      make_rsrc(a.partials + (static_cast<int64_t>(gridDim.x) + blockIdx.x) * a.N, static_cast<uint32_t>(a.N) * 4u);
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    const uint32_t o = k < chunks ? (k * kWideThreads + threadIdx.x) * VEC * 4u : kOutOfRange;
    if (a.partials_nt) {
      buf_store_f32<VEC, kNontemporal>(accw[k], rpw, o);
      buf_store_f32<VEC, kNontemporal>(accb[k], rpb, o);
    } else {
      buf_store_f32<VEC, kDefault>(accw[k], rpw, o);
      buf_store_f32<VEC, kDefault>(accb[k], rpb, o);
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side dispatch to the compiled instantiations.
// ---------------------------------------------------------------------------
template <typename S, int VEC, int ITERS>
hipError_t ln_fwd_inst(const RowPlan& p, const LnFwdArgs& a, hipStream_t s) {
  if constexpr (VEC * ITERS > lane_elems_cap(RowOp::kLnFwd, sizeof(S))) {
    return hipErrorInvalidValue;  // beyond the register model: never planned, not compiled
  } else {
    hipLaunchKernelGGL((layernorm_fwd_kernel<S, VEC, ITERS>), dim3(static_cast<unsigned>(p.grid)), dim3(p.threads()), 0,
                       s, a);
    return hipGetLastError();
  }
}

template <typename S, int VEC, int ITERS>
hipError_t ln_bwd_inst(const RowPlan& p, const LnBwdArgs& a, hipStream_t s) {
  if constexpr (VEC * ITERS > lane_elems_cap(RowOp::kLnBwd, sizeof(S))) {
    return hipErrorInvalidValue;  // beyond the register model: never planned, not compiled
  } else {
    const size_t lds = p.rpb > 1 ? 2 * static_cast<size_t>(a.N) * sizeof(float) : 0;
    if constexpr (bwd_needs_narrow_build(RowOp::kLnBwd, dtype_code<S>(), VEC, ITERS)) {
      // pipelined only in the build for workgroups of at most kNarrowThreads
      // threads, which the planner keeps to
      if (a.pipeline) {
        if (p.threads() > kNarrowThreads) return hipErrorInvalidValue;
        hipLaunchKernelGGL((layernorm_bwd_rows_kernel<S, VEC, ITERS, kNarrowThreads>), dim3(static_cast<unsigned>(p.grid)),
                           dim3(p.threads()), lds, s, a);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((layernorm_bwd_rows_kernel<S, VEC, ITERS, 1024>), dim3(static_cast<unsigned>(p.grid)),
                       dim3(p.threads()), lds, s, a);
    return hipGetLastError();
  }
}

template <typename S, int VEC>
hipError_t ln_fwd_vec(const RowPlan& p, const LnFwdArgs& a, hipStream_t s) {
  return pick_iters<LnFwdArgs, ln_fwd_inst<S, VEC, 1>, ln_fwd_inst<S, VEC, 2>, ln_fwd_inst<S, VEC, 4>,
                    ln_fwd_inst<S, VEC, 5>, ln_fwd_inst<S, VEC, 8>, ln_fwd_inst<S, VEC, 16>>(p, a, s);
}

template <typename S, int VEC>
hipError_t ln_bwd_vec(const RowPlan& p, const LnBwdArgs& a, hipStream_t s) {
  return pick_iters<LnBwdArgs, ln_bwd_inst<S, VEC, 1>, ln_bwd_inst<S, VEC, 2>, ln_bwd_inst<S, VEC, 4>,
                    ln_bwd_inst<S, VEC, 5>, ln_bwd_inst<S, VEC, 8>, ln_bwd_inst<S, VEC, 16>>(p, a, s);
}

template <typename S>
hipError_t ln_wide_fwd_s(const RowPlan& p, const LnFwdArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(p.grid)), block(kWideThreads);
  switch (p.vec) {
    case 1: hipLaunchKernelGGL((layernorm_fwd_wide_kernel<S, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((layernorm_fwd_wide_kernel<S, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((layernorm_fwd_wide_kernel<S, 4>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((layernorm_fwd_wide_kernel<S, 8>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename S>
hipError_t ln_wide_bwd_s(const RowPlan& p, const LnBwdArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(p.grid)), block(kWideThreads);
  switch (p.vec) {
    case 1: hipLaunchKernelGGL((layernorm_bwd_wide_kernel<S, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((layernorm_bwd_wide_kernel<S, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((layernorm_bwd_wide_kernel<S, 4>), grid, block, 0, s, a); break;
    case 8:
      // 16385-32768 elements: three or four 8192-element chunks
      static_assert(kLnWideHeldChunksMin == 3 && kLnWideHeldChunksMax == 4, "held-row instantiations");
      static_assert(kWideThreads * 16 == 16384, "a chunk of 16-byte vectors");
      if (a.chunks == 3) {
        hipLaunchKernelGGL((layernorm_bwd_wide_held_kernel<S, 3>), grid, block, kLnWideHeldLdsBytes(3), s, a);
      } else if (a.chunks == 4) {
        hipLaunchKernelGGL((layernorm_bwd_wide_held_kernel<S, 4>), grid, block, kLnWideHeldLdsBytes(4), s, a);
      } else {
        return hipErrorInvalidValue;  // never planned
      }
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ln_fwd_wide(int dtype, const RowPlan& p, const LnFwdArgs& a, hipStream_t s) {
  if (dtype == 1) return ln_wide_fwd_s<uint16_t>(p, a, s);
  if (dtype == 2) return ln_wide_fwd_s<_Float16>(p, a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_ln_bwd_wide(int dtype, const RowPlan& p, const LnBwdArgs& a, hipStream_t s) {
  if (dtype == 1) return ln_wide_bwd_s<uint16_t>(p, a, s);
  if (dtype == 2) return ln_wide_bwd_s<_Float16>(p, a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_ln_fwd(int dtype, const RowPlan& p, const LnFwdArgs& a, hipStream_t s) {
  if (dtype == 0) {
    switch (p.vec) {
      case 1: return ln_fwd_vec<float, 1>(p, a, s);
      case 2: return ln_fwd_vec<float, 2>(p, a, s);
      case 4: return ln_fwd_vec<float, 4>(p, a, s);
    }
  } else if (dtype == 1) {
    switch (p.vec) {
      case 1: return ln_fwd_vec<uint16_t, 1>(p, a, s);
      case 2: return ln_fwd_vec<uint16_t, 2>(p, a, s);
      case 4: return ln_fwd_vec<uint16_t, 4>(p, a, s);
      case 8: return ln_fwd_vec<uint16_t, 8>(p, a, s);
    }
  } else if (dtype == 2) {
    switch (p.vec) {
      case 1: return ln_fwd_vec<_Float16, 1>(p, a, s);
      case 2: return ln_fwd_vec<_Float16, 2>(p, a, s);
      case 4: return ln_fwd_vec<_Float16, 4>(p, a, s);
      case 8: return ln_fwd_vec<_Float16, 8>(p, a, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_ln_bwd_rows(int dtype, const RowPlan& p, const LnBwdArgs& a, hipStream_t s) {
  if (dtype == 0) {
    switch (p.vec) {
      case 1: return ln_bwd_vec<float, 1>(p, a, s);
      case 2: return ln_bwd_vec<float, 2>(p, a, s);
      case 4: return ln_bwd_vec<float, 4>(p, a, s);
    }
  } else if (dtype == 1) {
    switch (p.vec) {
      case 1: return ln_bwd_vec<uint16_t, 1>(p, a, s);
      case 2: return ln_bwd_vec<uint16_t, 2>(p, a, s);
      case 4: return ln_bwd_vec<uint16_t, 4>(p, a, s);
      case 8: return ln_bwd_vec<uint16_t, 8>(p, a, s);
    }
  } else if (dtype == 2) {
    switch (p.vec) {
      case 1: return ln_bwd_vec<_Float16, 1>(p, a, s);
      case 2: return ln_bwd_vec<_Float16, 2>(p, a, s);
      case 4: return ln_bwd_vec<_Float16, 4>(p, a, s);
      case 8: return ln_bwd_vec<_Float16, 8>(p, a, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace rmsn
