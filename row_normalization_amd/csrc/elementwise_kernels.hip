// gfx950 (CDNA4) kernels for the two elementwise ops of the Unsloth kernel
// walkthrough ("02 · 手写 Triton kernel:RMSNorm / RoPE / SwiGLU"):
//  - RoPE (section 4): in-place rotation of each (first-half, second-half)
//    pair of a head by its token's angle, q1' = q1 c - q2 s, q2' = q2 c + q1 s;
//    the backward is the same kernel with sin negated.
//  - SwiGLU (section 5): forward h = T(T(silu(e)) g); backward h, df = dh T(f)
//    and de = dh g s (1 + e (1 - s)) from dh, e and g in one pass.
//
// Both are pure streaming: every element is read once and written once, with
// a few flops in between, so the design is about moving 16-byte vectors
// through HBM: raw buffer loads and stores through descriptors whose range
// masks the tails (no branches around memory operations), all of a lane's
// loads issued before its arithmetic, nontemporal cache policy for the
// streamed operands.  Arithmetic is fp32; outputs are rounded once per the
// formulas above.  An output may be one of the inputs (in place): every lane
// reads all of its input elements before it writes the same elements, and no
// other lane touches them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "launch.h"

namespace rmsn {
namespace {
using namespace dev;

// ---------------------------------------------------------------------------
// RoPE.  Work item (token t, head group hg, vector v): the lane loads the
// cos/sin values of its vector once and rotates the same vector pair of
// kRopeGroup heads (the page's grouping of four heads per program, which
// spreads one table load over four heads).  v varies fastest, so the lanes of
// a wave cover whole 128-byte segments of a head half.
// ---------------------------------------------------------------------------
template <typename S, int VEC>
__global__ __launch_bounds__(kEltThreads) void rope_kernel(const RopeArgs a) {
  const int64_t item = static_cast<int64_t>(blockIdx.x) * kEltThreads + threadIdx.x;
  if (item >= a.items) return;
  const int64_t per_token = static_cast<int64_t>(a.groups) * a.nvh;
  const int64_t t = item / per_token;
  const int rem = static_cast<int>(item - t * per_token);
  const int hg = rem / a.nvh;
  const int v = rem - hg * a.nvh;

  int64_t pos;
  if (a.positions) {
    pos = a.positions[t];
  } else {
    pos = t % a.seq_len;
  }
  // positions outside the table read zeros (out of the descriptors' range)
  const uint32_t table_bytes = static_cast<uint32_t>(a.table_rows * a.half) * 4u;
  const bool in_table = pos >= 0 && pos < a.table_rows;
  const uint32_t toff = in_table ? (static_cast<uint32_t>(pos) * static_cast<uint32_t>(a.half) +
                                    static_cast<uint32_t>(v * VEC)) * 4u
                                 : kOutOfRange;
  float c[VEC], s[VEC];
  buf_load_f32<VEC, kDefault>(c, make_rsrc(a.cos, table_bytes), toff);
  buf_load_f32<VEC, kDefault>(s, make_rsrc(a.sin, table_bytes), toff);

  // one descriptor over the token's heads: heads past the last read zero and
  // are not written
  const uint32_t head_bytes = static_cast<uint32_t>(a.half) * 2u * sizeof(S);
  const Rsrc rq = make_rsrc(static_cast<S*>(a.q) + t * a.stride, static_cast<uint32_t>(a.heads) * head_bytes);
  const uint32_t half_bytes = static_cast<uint32_t>(a.half) * sizeof(S);
  const uint32_t base = static_cast<uint32_t>(hg * kRopeGroup) * head_bytes + static_cast<uint32_t>(v * VEC) * sizeof(S);

  Pack<S, VEC> q1[kRopeGroup], q2[kRopeGroup];
#pragma unroll
  for (int k = 0; k < kRopeGroup; ++k) {
    q1[k] = buf_load<S, VEC, kNontemporal>(rq, base + k * head_bytes);
    q2[k] = buf_load<S, VEC, kNontemporal>(rq, base + k * head_bytes + half_bytes);
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) s[e] *= a.sin_sign;
#pragma unroll
  for (int k = 0; k < kRopeGroup; ++k) {
    float o1[VEC], o2[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const float x1 = q1[k].get(e), x2 = q2[k].get(e);
      o1[e] = fmaf(x1, c[e], -x2 * s[e]);
      o2[e] = fmaf(x2, c[e], x1 * s[e]);
    }
    buf_store<S, VEC, kNontemporal>(round_pack<S, VEC>(o1), rq, base + k * head_bytes);
    buf_store<S, VEC, kNontemporal>(round_pack<S, VEC>(o2), rq, base + k * head_bytes + half_bytes);
  }
}

// ---------------------------------------------------------------------------
// SwiGLU.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float sigmoid_f32(float e) { return 1.0f / (1.0f + __expf(-e)); }

template <typename S, int VEC>
__global__ __launch_bounds__(kEltThreads) void swiglu_fwd_kernel(const SwigluArgs a) {
  constexpr uint32_t kPack = Pack<S, VEC>::kBytes;
  for (int64_t b = blockIdx.x; b < a.blocks; b += gridDim.x) {
    const int64_t row = b / a.tiles;
    const int tile = static_cast<int>(b - row * a.tiles);
    const int64_t off = row * a.stride;
    const uint32_t row_bytes = static_cast<uint32_t>(row == a.M - 1 ? a.last_row_elems : a.N) * sizeof(S);
    const Rsrc re = make_rsrc(static_cast<const S*>(a.e) + off, row_bytes);
    const Rsrc rg = make_rsrc(static_cast<const S*>(a.g) + off, row_bytes);
    const Rsrc rh = make_rsrc(static_cast<S*>(a.h) + off, row_bytes);
    const uint32_t v0 = static_cast<uint32_t>(tile) * kSwigluUnroll * kEltThreads + threadIdx.x;
    Pack<S, VEC> ev[kSwigluUnroll], gv[kSwigluUnroll];
#pragma unroll
    for (int u = 0; u < kSwigluUnroll; ++u) {
      ev[u] = buf_load<S, VEC, kNontemporal>(re, (v0 + u * kEltThreads) * kPack);
      gv[u] = buf_load<S, VEC, kNontemporal>(rg, (v0 + u * kEltThreads) * kPack);
    }
#pragma unroll
    for (int u = 0; u < kSwigluUnroll; ++u) {
      float o[VEC];
#pragma unroll
      for (int k = 0; k < VEC; ++k) {
        const float e = ev[u].get(k);
        const float f = round_to<S>(e * sigmoid_f32(e));  // f cast to the I/O type before the product
        o[k] = f * gv[u].get(k);
      }
      buf_store<S, VEC, kNontemporal>(round_pack<S, VEC>(o), rh, (v0 + u * kEltThreads) * kPack);
    }
  }
}

template <typename S, int VEC>
__global__ __launch_bounds__(kEltThreads) void swiglu_bwd_kernel(const SwigluArgs a) {
  constexpr uint32_t kPack = Pack<S, VEC>::kBytes;
  for (int64_t b = blockIdx.x; b < a.blocks; b += gridDim.x) {
    const int64_t row = b / a.tiles;
    const int tile = static_cast<int>(b - row * a.tiles);
    const int64_t off = row * a.stride;
    const uint32_t row_bytes = static_cast<uint32_t>(row == a.M - 1 ? a.last_row_elems : a.N) * sizeof(S);
    const Rsrc rdh = make_rsrc(static_cast<const S*>(a.dh) + off, row_bytes);
    const Rsrc re = make_rsrc(static_cast<const S*>(a.e) + off, row_bytes);
    const Rsrc rg = make_rsrc(static_cast<const S*>(a.g) + off, row_bytes);
    const uint32_t v0 = static_cast<uint32_t>(tile) * kSwigluUnroll * kEltThreads + threadIdx.x;
    Pack<S, VEC> dv[kSwigluUnroll], ev[kSwigluUnroll], gv[kSwigluUnroll];
#pragma unroll
    for (int u = 0; u < kSwigluUnroll; ++u) {
      const uint32_t o = (v0 + u * kEltThreads) * kPack;
      dv[u] = buf_load<S, VEC, kNontemporal>(rdh, o);
      ev[u] = buf_load<S, VEC, kNontemporal>(re, o);
      gv[u] = buf_load<S, VEC, kNontemporal>(rg, o);
    }
    // every input element of this lane is in registers before any output is written
    const Rsrc rh = make_rsrc(static_cast<S*>(a.h) + off, row_bytes);
    const Rsrc rdf = make_rsrc(static_cast<S*>(a.df) + off, row_bytes);
    const Rsrc rde = make_rsrc(static_cast<S*>(a.de) + off, row_bytes);
#pragma unroll
    for (int u = 0; u < kSwigluUnroll; ++u) {
      float oh[VEC], odf[VEC], ode[VEC];
#pragma unroll
      for (int k = 0; k < VEC; ++k) {
        const float d = dv[u].get(k), e = ev[u].get(k), g = gv[u].get(k);
        const float sg = sigmoid_f32(e);
        const float f = round_to<S>(e * sg);
        oh[k] = f * g;
        odf[k] = d * f;
        ode[k] = d * g * (sg * fmaf(e, 1.0f - sg, 1.0f));
      }
      const uint32_t o = (v0 + u * kEltThreads) * kPack;
      buf_store<S, VEC, kNontemporal>(round_pack<S, VEC>(oh), rh, o);
      buf_store<S, VEC, kNontemporal>(round_pack<S, VEC>(odf), rdf, o);
      buf_store<S, VEC, kNontemporal>(round_pack<S, VEC>(ode), rde, o);
    }
  }
}

// Grid of the elementwise launches: one item (or block) per thread group, capped.
constexpr int64_t kEltGridMax = int64_t(1) << 20;

template <typename S, int VEC>
hipError_t rope_inst(const RopeArgs& a, hipStream_t s) {
  const int64_t grid = (a.items + kEltThreads - 1) / kEltThreads;
  hipLaunchKernelGGL((rope_kernel<S, VEC>), dim3(static_cast<unsigned>(grid)), dim3(kEltThreads), 0, s, a);
  return hipGetLastError();
}

template <typename S, int VEC, bool BWD>
hipError_t swiglu_inst(const SwigluArgs& a, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>(a.blocks < kEltGridMax ? a.blocks : kEltGridMax);
  if constexpr (BWD) {
    hipLaunchKernelGGL((swiglu_bwd_kernel<S, VEC>), dim3(grid), dim3(kEltThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((swiglu_fwd_kernel<S, VEC>), dim3(grid), dim3(kEltThreads), 0, s, a);
  }
  return hipGetLastError();
}

template <typename S>
hipError_t rope_s(int vec, const RopeArgs& a, hipStream_t s) {
  switch (vec) {
    case 1: return rope_inst<S, 1>(a, s);
    case 2: return rope_inst<S, 2>(a, s);
    case 4: return rope_inst<S, 4>(a, s);
    case 8:
      if constexpr (sizeof(S) == 2) return rope_inst<S, 8>(a, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <typename S, bool BWD>
hipError_t swiglu_s(int vec, const SwigluArgs& a, hipStream_t s) {
  switch (vec) {
    case 1: return swiglu_inst<S, 1, BWD>(a, s);
    case 2: return swiglu_inst<S, 2, BWD>(a, s);
    case 4: return swiglu_inst<S, 4, BWD>(a, s);
    case 8:
      if constexpr (sizeof(S) == 2) return swiglu_inst<S, 8, BWD>(a, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <bool BWD>
hipError_t swiglu_dispatch(int dtype, int vec, const SwigluArgs& a, hipStream_t s) {
  switch (dtype) {
    case 0: return swiglu_s<float, BWD>(vec, a, s);
    case 1: return swiglu_s<uint16_t, BWD>(vec, a, s);
    case 2: return swiglu_s<_Float16, BWD>(vec, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_rope(int dtype, int vec, const RopeArgs& a, hipStream_t s) {
  switch (dtype) {
    case 0: return rope_s<float>(vec, a, s);
    case 1: return rope_s<uint16_t>(vec, a, s);
    case 2: return rope_s<_Float16>(vec, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_swiglu_fwd(int dtype, int vec, const SwigluArgs& a, hipStream_t s) {
  return swiglu_dispatch<false>(dtype, vec, a, s);
}

hipError_t launch_swiglu_bwd(int dtype, int vec, const SwigluArgs& a, hipStream_t s) {
  return swiglu_dispatch<true>(dtype, vec, a, s);
}

}  // namespace rmsn
