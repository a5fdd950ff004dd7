// Host side of the RoPE and SwiGLU C ABIs (include/rope.h, include/swiglu.h):
// argument validation, the choice of vector width, and the extern "C" entry
// points.  Validation is plain host arithmetic (no HIP call) and finishes
// before anything is launched; on failure nothing is written.
#include <cstdint>
#include <limits>

#include "host_plan.h"
#include "launch.h"
#include "rope.h"
#include "swiglu.h"

namespace rmsn {
namespace {

bool valid_dtype(int dtype) { return dtype == RMSNORM_F32 || dtype == RMSNORM_BF16 || dtype == RMSNORM_F16; }

// ---------------------------------------------------------------------------
// RoPE
// ---------------------------------------------------------------------------
constexpr int64_t kRopeHeadDimMax = 1024;
constexpr int64_t kRopeTokenElemsMax = int64_t(1) << 24;  // heads * head_dim
constexpr int64_t kRopeTableMax = int64_t(1) << 28;       // table_rows * head_dim / 2

int rope(void* q, int64_t tokens, int64_t heads, int64_t head_dim, int64_t token_stride, const float* cos,
         const float* sin, int64_t table_rows, const int32_t* positions, int64_t seq_len, int dtype, float sin_sign,
         hipStream_t stream) {
  if (!valid_dtype(dtype)) return RMSNORM_E_DTYPE;
  if (tokens < 0 || tokens > RMSNORM_M_MAX || heads < 1 || head_dim < 2 || head_dim > kRopeHeadDimMax ||
      head_dim % 2 || heads > kRopeTokenElemsMax / head_dim || table_rows < 1 ||
      table_rows > kRopeTableMax / (head_dim / 2))
    return RMSNORM_E_SHAPE;
  if (!positions && (seq_len < 1 || seq_len > table_rows)) return RMSNORM_E_SHAPE;
  if (token_stride < heads * head_dim) return RMSNORM_E_STRIDE;
  // byte offsets of every token must fit int64 (as for the row-wise ops)
  if (tokens > 0 && token_stride > (std::numeric_limits<int64_t>::max() / 8) / tokens) return RMSNORM_E_SHAPE;
  if (tokens == 0) return RMSNORM_OK;
  if (!q || !cos || !sin) return RMSNORM_E_NULL;
  const int es = elsize(dtype);
  if (!aligned(q, es) || !aligned(cos, 4) || !aligned(sin, 4) || (positions && !aligned(positions, 4)))
    return RMSNORM_E_ALIGN;
  const int64_t half = head_dim / 2;
  const Span sq = span(q, ((tokens - 1) * token_stride + heads * head_dim) * es);
  if (overlap(sq, span(cos, table_rows * half * 4)) || overlap(sq, span(sin, table_rows * half * 4)) ||
      (positions && overlap(sq, span(positions, tokens * 4))))
    return RMSNORM_E_ALIAS;

  // widest vector (<= 16 bytes of q) that the half-head, the token stride and
  // every base pointer allow; the tables are read in fp32 vectors of the same
  // element count (16-byte pieces)
  int vec = 16 / es;
  while (vec > 1 && (half % vec || token_stride % vec || !aligned(q, int64_t(vec) * es) ||
                     !aligned(cos, std::min<int64_t>(16, vec * 4)) || !aligned(sin, std::min<int64_t>(16, vec * 4))))
    vec /= 2;
  RopeArgs a{};
  a.q = q;
  a.cos = cos;
  a.sin = sin;
  a.positions = positions;
  a.tokens = tokens;
  a.stride = token_stride;
  a.table_rows = table_rows;
  a.seq_len = positions ? 1 : seq_len;
  a.heads = static_cast<int32_t>(heads);
  a.half = static_cast<int32_t>(half);
  a.groups = static_cast<int32_t>(ceil_div(heads, kRopeGroup));
  a.nvh = static_cast<int32_t>(half / vec);
  a.items = tokens * a.groups * a.nvh;
  a.sin_sign = sin_sign;
  // one thread per item: the launch's work-item count (blocks x threads)
  // must fit the 32-bit grid size of a dispatch
  if (ceil_div(a.items, kEltThreads) * kEltThreads > (int64_t(1) << 32) - 1) return RMSNORM_E_SHAPE;
  return hip_status(launch_rope(dtype, vec, a, stream));
}

// ---------------------------------------------------------------------------
// SwiGLU
// ---------------------------------------------------------------------------
constexpr int64_t kSwigluNMax = int64_t(1) << 26;

int check_swiglu_shape(int64_t M, int64_t N, int64_t stride, int dtype) {
  if (!valid_dtype(dtype)) return RMSNORM_E_DTYPE;
  if (M < 0 || M > RMSNORM_M_MAX || N < 1 || N > kSwigluNMax) return RMSNORM_E_SHAPE;
  if (stride < N) return RMSNORM_E_STRIDE;
  if (M > 0 && stride > (std::numeric_limits<int64_t>::max() / 8) / M) return RMSNORM_E_SHAPE;
  return RMSNORM_OK;
}

// Outputs may each be exactly one of the inputs (same pointer); otherwise an
// output must not share a byte with an input, and no two outputs may share a
// byte (exact row-segment test: interleaved views of one buffer are fine).
int check_outputs(std::initializer_list<const void*> ins, std::initializer_list<const void*> outs, int64_t M,
                  int64_t N, int64_t stride, int es) {
  const void* const* o = outs.begin();
  for (size_t a = 0; a < outs.size(); ++a) {
    for (const void* i : ins)
      if (o[a] != i && matrices_overlap(o[a], i, M, N, stride, es)) return RMSNORM_E_ALIAS;
    for (size_t b = a + 1; b < outs.size(); ++b)
      if (matrices_overlap(o[a], o[b], M, N, stride, es)) return RMSNORM_E_ALIAS;
  }
  return RMSNORM_OK;
}

SwigluArgs swiglu_args(const void* e, const void* g, const void* dh, void* h, void* df, void* de, int64_t M,
                       int64_t N, int64_t stride, int vec) {
  int64_t last = N;
  if (stride == N && M * N > kSwigluFlatRow) {
    // dense: the same elements as rows of kSwigluFlatRow (a multiple of every
    // tile length, and of vec, so the last row's length is one as well)
    const int64_t total = M * N;
    M = ceil_div(total, kSwigluFlatRow);
    N = stride = kSwigluFlatRow;
    last = total - (M - 1) * kSwigluFlatRow;
  }
  SwigluArgs a{};
  a.e = e;
  a.g = g;
  a.dh = dh;
  a.h = h;
  a.df = df;
  a.de = de;
  a.M = M;
  a.stride = stride;
  a.N = static_cast<int32_t>(N);
  a.tiles = static_cast<int32_t>(ceil_div(N / vec, int64_t(kSwigluUnroll) * kEltThreads));
  a.blocks = M * a.tiles;
  a.last_row_elems = last;
  return a;
}

}  // namespace
}  // namespace rmsn

using namespace rmsn;

extern "C" {

int rope_fwd(void* q, int64_t tokens, int64_t heads, int64_t head_dim, int64_t token_stride, const float* cos,
             const float* sin, int64_t table_rows, const int32_t* positions, int64_t seq_len, int dtype,
             hipStream_t stream) {
  return rope(q, tokens, heads, head_dim, token_stride, cos, sin, table_rows, positions, seq_len, dtype, 1.0f,
              stream);
}

int rope_bwd(void* dq, int64_t tokens, int64_t heads, int64_t head_dim, int64_t token_stride, const float* cos,
             const float* sin, int64_t table_rows, const int32_t* positions, int64_t seq_len, int dtype,
             hipStream_t stream) {
  return rope(dq, tokens, heads, head_dim, token_stride, cos, sin, table_rows, positions, seq_len, dtype, -1.0f,
              stream);
}

int swiglu_fwd(const void* e, const void* g, void* h, int64_t M, int64_t N, int64_t row_stride, int dtype,
               hipStream_t stream) {
  int st = check_swiglu_shape(M, N, row_stride, dtype);
  if (st) return st;
  if (M == 0) return RMSNORM_OK;
  if (!e || !g || !h) return RMSNORM_E_NULL;
  const int es = elsize(dtype);
  if (!aligned(e, es) || !aligned(g, es) || !aligned(h, es)) return RMSNORM_E_ALIGN;
  st = check_outputs({e, g}, {h}, M, N, row_stride, es);
  if (st) return st;
  const int vec = choose_vec(dtype, N, row_stride, {e, g, h});
  return hip_status(launch_swiglu_fwd(dtype, vec, swiglu_args(e, g, nullptr, h, nullptr, nullptr, M, N, row_stride, vec),
                                      stream));
}

int swiglu_bwd(const void* dh, const void* e, const void* g, void* h, void* df, void* de, int64_t M, int64_t N,
               int64_t row_stride, int dtype, hipStream_t stream) {
  int st = check_swiglu_shape(M, N, row_stride, dtype);
  if (st) return st;
  if (M == 0) return RMSNORM_OK;
  if (!dh || !e || !g || !h || !df || !de) return RMSNORM_E_NULL;
  const int es = elsize(dtype);
  for (const void* p : {dh, e, g, static_cast<const void*>(h), static_cast<const void*>(df),
                        static_cast<const void*>(de)})
    if (!aligned(p, es)) return RMSNORM_E_ALIGN;
  st = check_outputs({dh, e, g}, {h, df, de}, M, N, row_stride, es);
  if (st) return st;
  const int vec = choose_vec(dtype, N, row_stride, {dh, e, g, h, df, de});
  return hip_status(launch_swiglu_bwd(dtype, vec, swiglu_args(e, g, dh, h, df, de, M, N, row_stride, vec), stream));
}

}  // extern "C"
