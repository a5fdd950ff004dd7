// Device-side building blocks shared by every kernel of the library (RMSNorm,
// LayerNorm, RoPE, SwiGLU): packed vectors, raw-buffer access with hardware
// range checks, rounding to the I/O types, the wave / row-group reductions
// and the dispatch helper.  Included by the .hip files only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "launch.h"

namespace rmsn {
namespace dev {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t Rsrc;

// The dtype code (rmsnorm_dtype) of a storage type: float, uint16_t (bf16
// bits), _Float16.
template <typename S>
constexpr int dtype_code() {
  return sizeof(S) == 4 ? 0 : std::is_same<S, _Float16>::value ? 2 : 1;
}

// An LDS table of nvec vectors of VEC floats (the LayerNorm backward's
// row-group combine), laid out as VEC / 4 planes of nvec four-float cells (one plane of VEC-float cells for VEC < 4):
// a wave's 16-byte accesses then cover consecutive addresses, free of bank
// conflicts, where VEC = 8 consecutive floats per lane (a 32-byte lane
// stride) conflict.  Measured on MI355X: LayerNorm fp16 backward 1-5 %
// faster (4096 x 1024-8192, 1151 x 8192); the RMSNorm combine, whose
// conflicts were few, was 1-5 % slower with it at N = 1024 and keeps VEC
// consecutive floats per vector.
// Cells are moved as whole 16-byte (8-, 4-byte) LDS accesses: written
// element by element, with the other table's stores in between, they would
// become single-float accesses, as the compiler cannot tell that the two
// tables do not overlap.
template <int VEC>
__device__ __forceinline__ void comb_store(float* table, int v, int nvec, const float (&x)[VEC]) {
  constexpr int kCell = VEC < 4 ? VEC : 4;
  typedef float cell_t __attribute__((ext_vector_type(kCell)));
#pragma unroll
  for (int h = 0; h < VEC / kCell; ++h) {
    cell_t c;
#pragma unroll
    for (int e = 0; e < kCell; ++e) c[e] = x[h * kCell + e];
    *reinterpret_cast<cell_t*>(table + (h * nvec + v) * kCell) = c;
  }
}

template <int VEC>
__device__ __forceinline__ void comb_load(const float* table, int v, int nvec, float (&x)[VEC]) {
  constexpr int kCell = VEC < 4 ? VEC : 4;
  typedef float cell_t __attribute__((ext_vector_type(kCell)));
#pragma unroll
  for (int h = 0; h < VEC / kCell; ++h) {
    const cell_t c = *reinterpret_cast<const cell_t*>(table + (h * nvec + v) * kCell);
#pragma unroll
    for (int e = 0; e < kCell; ++e) x[h * kCell + e] = c[e];
  }
}

// Word 3 of a raw (untyped, stride 0) buffer descriptor on the gfx9 family:
// 32-bit data format; the range check is then offset against the byte count.
constexpr int kRsrcWord3 = 0x00020000;
// Cache-policy operand of buffer instructions: 0 = default, 2 = nontemporal
// (streamed, not kept).  (Measured on MI355X: adding the device-scope bit to
// the row kernels' nontemporal stores, so they are written through L2, made
// them 0.2-1.9 % slower in interleaved comparisons.)
constexpr int kDefault = 0;
constexpr int kNontemporal = 2;

// A descriptor for `bytes` bytes at `base`; accesses at or past `bytes` read
// zero and write nothing.
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kRsrcWord3);
}

// VEC consecutive elements with the storage type S (float; uint16_t for bf16
// bits; _Float16), aligned to their full width so one load/store moves them.  They
// are held as 32-bit words (two bf16 per word) whenever the pack is at least
// 4 bytes wide.
template <typename S, int VEC>
struct alignas(sizeof(S) * VEC) Pack {
  static constexpr int kBytes = int(sizeof(S)) * VEC;
  static constexpr int kWords = kBytes >= 4 ? kBytes / 4 : 1;
  typedef typename std::conditional<(kBytes >= 4), uint32_t, uint16_t>::type Word;
  Word w[kWords];

  // element e as fp32 (exact: bf16 bits move to the top half of an fp32;
  // fp16 converts in hardware)
  __device__ __forceinline__ float get(int e) const {
    if constexpr (sizeof(S) == 4) {
      return __builtin_bit_cast(float, w[e]);
    } else if constexpr (std::is_same<S, _Float16>::value) {
      const uint32_t word = kBytes == 2 ? static_cast<uint32_t>(w[0]) : static_cast<uint32_t>(w[e >> 1]);
      const uint16_t h = static_cast<uint16_t>((e & 1) ? (word >> 16) : word);
      return static_cast<float>(__builtin_bit_cast(_Float16, h));
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

// One pack from a buffer at byte offset `off`.  The whole offset goes in the
// instruction's vector offset, which the range check covers (the scalar
// offset operand is left at zero: it is added to the address but not checked).
template <typename S, int VEC, int AUX>
__device__ __forceinline__ Pack<S, VEC> buf_load(Rsrc r, uint32_t off) {
  typedef Pack<S, VEC> P;
  if constexpr (P::kBytes == 16) {
    return __builtin_bit_cast(P, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
  } else if constexpr (P::kBytes == 8) {
    return __builtin_bit_cast(P, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX));
  } else if constexpr (P::kBytes == 4) {
    return __builtin_bit_cast(P, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX));
  } else {
    return __builtin_bit_cast(P, __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, AUX));
  }
}

template <typename S, int VEC, int AUX>
__device__ __forceinline__ void buf_store(const Pack<S, VEC>& p, Rsrc r, uint32_t off) {
  typedef Pack<S, VEC> P;
  if constexpr (P::kBytes == 16) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, p), r, off, 0, AUX);
  } else if constexpr (P::kBytes == 8) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, p), r, off, 0, AUX);
  } else if constexpr (P::kBytes == 4) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, p), r, off, 0, AUX);
  } else {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, p), r, off, 0, AUX);
  }
}

// VEC fp32 values at byte offset `off`, in stores of at most 16 bytes.
template <int VEC, int AUX>
__device__ __forceinline__ void buf_store_f32(const float (&v)[VEC], Rsrc r, uint32_t off) {
  if constexpr (VEC > 4) {
#pragma unroll
    for (int k = 0; k < VEC; k += 4) {
      const u32x4_t q = {__builtin_bit_cast(uint32_t, v[k]), __builtin_bit_cast(uint32_t, v[k + 1]),
                         __builtin_bit_cast(uint32_t, v[k + 2]), __builtin_bit_cast(uint32_t, v[k + 3])};
      __builtin_amdgcn_raw_buffer_store_b128(q, r, off + k * 4u, 0, AUX);
    }
  } else {
    Pack<float, VEC> p;
#pragma unroll
    for (int e = 0; e < VEC; ++e) p.w[e] = __builtin_bit_cast(uint32_t, v[e]);
    buf_store<float, VEC, AUX>(p, r, off);
  }
}

// VEC fp32 values from byte offset `off`, in loads of at most 16 bytes.
template <int VEC, int AUX>
__device__ __forceinline__ void buf_load_f32(float (&v)[VEC], Rsrc r, uint32_t off) {
  if constexpr (VEC > 4) {
#pragma unroll
    for (int k = 0; k < VEC; k += 4) {
      // through a 4-float pack, as buf_load does: an implicit conversion of
      // the builtin's vector result to u32x4_t compiles to a splat of its
      // first element
      const Pack<float, 4> q = buf_load<float, 4, AUX>(r, off + k * 4u);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[k + j] = q.get(j);
    }
  } else {
    const Pack<float, VEC> p = buf_load<float, VEC, AUX>(r, off);
#pragma unroll
    for (int e = 0; e < VEC; ++e) v[e] = p.get(e);
  }
}

// Byte offset that is out of range of every descriptor made here (their
// ranges are below 2^31 bytes).  It sits at 2^31, so a multi-piece access
// (a 32-byte fp32 vector read as two 16-byte loads) adds its piece offsets
// to it without wrapping back into range.
constexpr uint32_t kOutOfRange = 0x80000000u;

// Round VEC fp32 values once (to nearest even; gfx950 converts bf16 and fp16
// pairs in one instruction each) to the storage type S.
template <typename S, int VEC>
__device__ __forceinline__ Pack<S, VEC> round_pack(const float (&o)[VEC]) {
  typedef typename std::conditional<std::is_same<S, _Float16>::value, _Float16, __bf16>::type H;
  typedef H h2_t __attribute__((ext_vector_type(2)));
  Pack<S, VEC> p;
  if constexpr (sizeof(S) == 4) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) p.w[e] = __builtin_bit_cast(uint32_t, o[e]);
  } else if constexpr (VEC == 1) {
    p.w[0] = __builtin_bit_cast(uint16_t, static_cast<H>(o[0]));
  } else {
#pragma unroll
    for (int e = 0; e < VEC; e += 2) {
      const f32x2_t f = {o[e], o[e + 1]};
      p.w[e >> 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, h2_t));
    }
  }
  return p;
}

// v rounded to the storage type S and back (the value a tensor of type S
// would hold); identity for fp32.
template <typename S>
__device__ __forceinline__ float round_to(float v) {
  if constexpr (sizeof(S) == 4) {
    return v;
  } else if constexpr (std::is_same<S, _Float16>::value) {
    return static_cast<float>(static_cast<_Float16>(v));
  } else {
    return static_cast<float>(static_cast<__bf16>(v));
  }
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

// Two sums per row group (for instance the two row sums of the LayerNorm
// backward) through one barrier; slots double-buffered by step parity like
// group_sum.
__device__ __forceinline__ void group_sum2(float& a, float& b, float (*red)[2][kMaxBlockWaves], int64_t step, int wave,
                                           int group, int wpr, int lane) {
  float(*slot)[kMaxBlockWaves] = red[step & 1];
  if (lane == 0) {
    slot[0][wave] = a;
    slot[1][wave] = b;
  }
  __syncthreads();
  float ta = 0.f, tb = 0.f;
  for (int k = 0; k < wpr; ++k) {
    ta += slot[0][group * wpr + k];
    tb += slot[1][group * wpr + k];
  }
  a = ta;
  b = tb;
}

// Where a lane sits: its wave (uniform, in a scalar register), the row group
// of the wave and the wave within the group.
struct Lane {
  int lane, wave, group, wv;
  __device__ __forceinline__ explicit Lane(int wpr) {
    lane = threadIdx.x & (kWave - 1);
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    group = wave / wpr;
    wv = wave - group * wpr;
  }
  // Two ways to give a row group's lanes the row's column vectors:
  // first_vec() + i * wpr * kWave (iteration-major: iteration i of all the
  // group's waves covers one contiguous stretch of the row) and
  // wave_vec<ITERS>(i) (wave-major: each wave owns ITERS * kWave contiguous
  // vectors).  The RMSNorm backward uses the wave-major order (measured on
  // MI355X: 1-3 % faster row passes, fp32 8192 x 8192 137.0 -> 132.7 us);
  // the forwards and the LayerNorm backward measured no better with it and
  // keep the iteration-major one.
  __device__ __forceinline__ uint32_t first_vec() const { return static_cast<uint32_t>(wv * kWave + lane); }
  template <int ITERS>
  __device__ __forceinline__ int wave_vec(int i) const { return (wv * ITERS + i) * kWave + lane; }
};

// Row handled by row group `group` of this workgroup at step `step` (of
// `row_iters`): at each step the workgroups cover consecutive rows, so the
// rows in flight across the chip form one compact window.
__device__ __forceinline__ int64_t row_of(int64_t step, int64_t row_iters, int rpb, int group) {
  (void)row_iters;
  return (step * gridDim.x + blockIdx.x) * rpb + group;
}

// Host-side dispatch from a plan's vectors-per-lane count to the compiled
// instantiation (one launcher per entry of kItersSet).
template <typename Args, hipError_t (*L1)(const RowPlan&, const Args&, hipStream_t),
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

}  // namespace dev
}  // namespace rmsn
