// Host-side helpers shared by the RMSNorm and LayerNorm C ABIs: pointer and
// span checks, the choice of vector width and the launch plan of the row
// kernels.  Plain host arithmetic; no HIP calls.
#pragma once

#include <algorithm>
#include <cstdint>
#include <initializer_list>
#include <limits>
#include <tuple>

#include "launch.h"
#include "rmsnorm.h"

namespace rmsn {

// Launch shape.  A row group spans as many waves as it takes for each lane
// to hold kLaneVectors 16-byte vectors of every row operand; workgroups hold
// about kBlockWaves waves (several row groups when rows are short).  Measured
// on MI355X at M=16384, N=8192 bf16: two vectors per lane and eight waves per
// row beat both fewer, fatter lanes and whole-row-per-wave layouts, for the
// forward and the backward alike.
constexpr int kLaneVectors = 2;
constexpr int kBlockWaves = 8;
constexpr int kFwdRowWaves = 8;
// The backward grid is persistent: a whole number of workgroups on each of
// the 256 compute units (a power of two, so that every CU gets the same
// count), about kBwdResidentWaves waves per CU, every workgroup taking a fixed
// share of the rows.  Each workgroup writes one fp32 partial row of dgamma.
// (A grid that does not divide evenly over the CUs leaves a tail: 819
// workgroups for N = 5120 ran 20 % slower than 512.)
constexpr int64_t kComputeUnits = 256;
constexpr int64_t kBwdResidentWaves = 16;
// Upper bound on the backward grid, hence on the partial rows a workspace
// must hold (rmsnorm_bwd_workspace_bytes promises this many rows at most).
constexpr int64_t kBwdGridMax = 1024;
// The forward grid is not persistent; it is only capped so that the grid
// dimension stays small (rows beyond it are taken in further steps).
constexpr int64_t kFwdGridMax = 1 << 20;
constexpr int64_t kFwdPersistentMinSteps = 8;
constexpr int64_t kFwdPersistentMinWaves = 14;
constexpr int64_t kLnFwdPersistentMinWaves = 12;

inline int elsize(int dtype) { return dtype == RMSNORM_F32 ? 4 : 2; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline bool aligned(const void* p, int64_t bytes) { return reinterpret_cast<uintptr_t>(p) % static_cast<uintptr_t>(bytes) == 0; }

// [p, p + len) for a byte range; empty ranges never overlap.
struct Span {
  uintptr_t lo;
  uintptr_t len;
};
inline Span span(const void* p, int64_t bytes) { return {reinterpret_cast<uintptr_t>(p), static_cast<uintptr_t>(bytes)}; }
inline bool overlap(Span a, Span b) { return a.len && b.len && a.lo < b.lo + b.len && b.lo < a.lo + a.len; }

// Whether two [M, N] matrices of `es`-byte elements with the same row stride
// (S elements) at p and q share a byte.  Exact for the row-segment layout:
// with d = q - p in bytes, row r of p meets row r + k of q iff
// |d + k * S * es| < N * es, which (N <= S) can only hold for the two k
// around -d / (S * es).  Lets disjoint interleaved views (the two halves of a
// fused [M, 2N] buffer) through where a span test would not.
inline bool matrices_overlap(const void* p, const void* q, int64_t M, int64_t N, int64_t S, int es) {
  if (M == 0 || N == 0) return false;
  const int64_t d = static_cast<int64_t>(reinterpret_cast<uintptr_t>(q) - reinterpret_cast<uintptr_t>(p));
  const int64_t rowb = N * es, sb = S * es;
  // k1 = ceil(-d / sb): d + k1 * sb lies in [0, sb), d + (k1 - 1) * sb in [-sb, 0)
  int64_t k1 = -d / sb;
  if (-d % sb > 0) ++k1;
  for (int64_t k : {k1, k1 - 1}) {
    if (k < -(M - 1) || k > M - 1) continue;
    const int64_t v = d + k * sb;
    if (v > -rowb && v < rowb) return true;
  }
  return false;
}

inline int64_t matrix_bytes(int64_t M, int64_t N, int64_t stride, int dtype) {
  return M == 0 ? 0 : ((M - 1) * stride + N) * elsize(dtype);
}

// Shape and stride limits shared by every row operation (n_max: the longest
// row the operation takes).
inline int check_shape(int64_t M, int64_t N, int64_t stride, int64_t n_max = RMSNORM_N_MAX) {
  if (M < 0 || M > RMSNORM_M_MAX || N < 1 || N > n_max) return RMSNORM_E_SHAPE;
  if (stride < N) return RMSNORM_E_STRIDE;
  // element offsets must stay well inside int64 even for the last row
  if (M > 0 && stride > (std::numeric_limits<int64_t>::max() / 8) / M) return RMSNORM_E_SHAPE;
  return RMSNORM_OK;
}

// Widest vector (up to 16 bytes) that every pointer, N and the stride allow.
inline int choose_vec(int dtype, int64_t N, int64_t stride, std::initializer_list<const void*> ptrs) {
  const int es = elsize(dtype);
  for (int vec = 16 / es; vec > 1; vec /= 2) {
    bool ok = N % vec == 0 && stride % vec == 0;
    for (const void* p : ptrs) ok = ok && aligned(p, int64_t(vec) * es);
    if (ok) return vec;
  }
  return 1;
}

// Waves per row and vectors per lane.  Candidates: 1..16 waves per row, a
// compiled register-array length within the lane's register budget, no wave
// without work.  The smallest key wins, compared in this order:
//   1. one vector per lane in a row of more than two waves;
//   2. waste (covered minus real vectors) above a quarter of the row;
//   3. 16-bit I/O, forward: a row of more than kFwdRowWaves waves;
//   4. 16-bit I/O: distance from `target` vectors per lane, then waste;
//      fp32 I/O: waste, then distance from `target`;
//   5. fewer waves.
// Measured on MI355X (forward and backward, M = 4096 and 16384): one vector
// per lane in rows of 9-15 waves ran 15-40 % slower than two vectors in
// half as many waves with a partly empty last wave (e.g. bf16 16384 x 7680
// forward 129 -> 82 us), and in rows of 3-7 waves 4-27 % slower than two or
// four vectors even with more than a quarter of the vectors empty (bf16
// 16384 x 3200 as 4 x 2 instead of 7 x 1: forward 49.4 -> 37.2 us, backward
// 57.4 -> 51.5 us; 16384 x 2304 backward as 3 x 2 instead of 5 x 1: 49.1 ->
// 38.5 us; fp32 N = 704, 1100, 1600 alike); 16-bit rows of 10-16 waves in the
// forward 7-17 % slower than 5-8 waves with 4 vectors; for fp32 rows, where a
// vector holds half the elements, the least waste was within 2 % of the best
// shape and the 16-bit order up to 6 % slower.
inline bool row_shape(int64_t nvec, int iters_cap, int target, bool narrow, bool backward, int* wpr, int* iters) {
  bool found = false;
  std::tuple<bool, bool, bool, int64_t, int64_t, int> best{};
  for (int w = 1; w <= kMaxBlockWaves; ++w) {
    for (int it : kItersSet) {
      if (it > iters_cap || int64_t(it) * kWave * w < nvec) continue;
      if (w > 1 && int64_t(it) * kWave * (w - 1) >= nvec) continue;
      const int64_t waste = int64_t(it) * kWave * w - nvec;
      const int64_t dist = it > target ? it - target : target - it;
      const auto key = std::make_tuple(it == 1 && w > 2, waste * 4 > nvec, narrow && !backward && w > kFwdRowWaves,
                                       narrow ? dist : waste, narrow ? waste : dist, w);
      if (!found || key < best) {
        found = true;
        best = key;
        *wpr = w;
        *iters = it;
      }
    }
  }
  return found;
}

// Backward grids.  Where the pipelined row loop is compiled for the plan
// (a workgroup alone on its CU needs it to keep loads in flight through its
// barriers), the backward runs one workgroup per CU, of the row's own shape
// (about kBlockWaves waves), pipelined.  Measured on MI355X (interleaved
// comparison, full backward = row pass and column sum) against two
// workgroups per CU without the pipeline: RMSNorm bf16 16384 x 8192 (Gemma,
// in place) 2.2 % faster (the fwd + bwd step 1.5 %), 32768 x 5120 2.1 %,
// 16384 x 1024-6144 2.8-5.0 %, 32768 x 1024-8192 1.2-3.3 %, 65536 x 4096
// 1.1 %; fp32 8192 x 1024-4096 1.7-3.5 %, 16384 x 1024-4096 0.2-1.3 %;
// LayerNorm fp16 32768 x 1024-8192 2.2-4.6 % (6144: 0.8 % slower), fp32
// 16384 x 2048 and 4096 1.9 and 2.5 %.  (Two workgroups per CU also write
// twice the partial rows.)
// Each workgroup writes one fp32 partial row per weight (two for LayerNorm)
// after its last row step, which the column sum reads back: with `grid`
// workgroups, tables * grid * 4 bytes per column against 3 * M * es of row
// traffic.  Where that share exceeds kBwdWideShare, rows of 5-8 waves run
// two to a 16-wave workgroup (still one per CU): 5-7 waves alone on a CU keep
// too few loads in flight (LayerNorm fp16 4096 x 4608-6656 3-18 % slower,
// 8192 x 6144 10 %, RMSNorm bf16 2048 x 8192 6 % slower as one 8-wave
// workgroup).  With one workgroup per CU each takes at least kBwdMinSteps
// row steps while the grid keeps kBwdMinGridWaves waves (8 per CU), and the
// grid is then the fewest workgroups that keep the step count and those
// waves.
// Measured on MI355X against two workgroups per CU (interleaved comparison;
// full backward) where the partial rows weigh: LayerNorm fp16 at M = 4096,
// N = 1024-5120, 4-17 % faster (N = 1024 17 %, 2048 15 %, 4096 16 %), the
// chapter's 1151 x 8192 17 %, 8192 x 2048 12 %, fp32 4096 x 2048 10 %;
// RMSNorm bf16 4096 x 4096 10 %, 4096 x 3072 13 %, 8192 x 2048 6.5 %,
// 1151 x 8192 9 %, 700 x 16384 7 %.  Rows of 1-4 waves in 16-wave
// workgroups (4-16 row groups to combine) were 3-37 % slower, so they keep
// their shape; one workgroup per CU of fewer than kBwdMinGridWaves / 256
// waves was slower (4096 x 1024 with 128 workgroups of 8 waves: 13 %).
constexpr double kBwdWideShare = 0.03;
// The bf16 LayerNorm backward pipelines only in its build for workgroups of
// at most kNarrowThreads threads (launch.h): there, rows of 1-4 waves (in
// workgroups of 6-8 waves) and rows of 8 waves where the partial rows are
// light run one workgroup per CU, pipelined.  Measured on MI355X
// (interleaved comparison, full backward) against the plans below: 4096 x
// 1024-4096 9-15 % faster, 8192 x 2048 8 %, 16384 x 2048 and 4096 4.5 and
// 3 %, 32768 x 4096 1.5 %, 16384 x 8192 5 %; rows of 5-7 waves alone on a
// CU were slower (16384 x 5120 17 %, 16384 and 32768 x 6144 4-5 %) and keep
// the plans below.
// Where the pipelined loop is not compiled for the plan (narrower vectors;
// the bf16 LayerNorm rows above), only rows of 4-8 waves run one 16-wave
// workgroup per CU (two to four row groups keep each other's loads in
// flight), and only above kBwdWideShareUnpipelined.  Measured on MI355X,
// LayerNorm bf16 full backward: 4096 x 4096 (share 0.33) 9 %, 4096 x 8192
// (0.17) 3 %, 4096 x 6144 (0.17) 1.8 %, 1151 x 8192 (0.59) 21 % faster;
// 16384 x 6432 (0.042) 5 % slower; rows of 1-3 waves (4096 x 1024-3072, 16
// row groups to combine) 0.5-22 % slower, as was fp32 RMSNorm 4096 x 1001.
constexpr double kBwdWideShareUnpipelined = 0.1;
constexpr int64_t kBwdMinSteps = 4;
constexpr int64_t kBwdMinGridWaves = 2048;

inline bool bwd_partials_heavy(RowOp op, int64_t M, int es, int64_t grid, double share = kBwdWideShare) {
  const int tables = op == RowOp::kLnBwd ? 2 : 1;
  return static_cast<double>(tables) * static_cast<double>(grid) * 4.0 > share * 3.0 * static_cast<double>(M) * es;
}

// Row shapes the rule above does not pick, where an interleaved comparison on
// MI355X found another shape faster.  An entry applies to the operations in
// `ops`, elements of `es` bytes (0: either), vectors of `vbytes` bytes (0:
// any width), rows of lo..hi vectors, and only where the rule's own shape is
// from_wpr x from_iters; such a row then runs as wpr x iters (waves x vectors
// per lane).  Every entry stays within the register model (vectors per lane
// at most the operation's cap for its vector width, checked for all widths
// by tests/native/plan_check.cpp).
constexpr unsigned op_bit(RowOp op) { return 1u << static_cast<int>(op); }
constexpr unsigned kFwdOps = op_bit(RowOp::kRmsFwd) | op_bit(RowOp::kLnFwd);
constexpr unsigned kBwdOps = op_bit(RowOp::kRmsBwd) | op_bit(RowOp::kLnBwd);
struct ShapeOverride {
  unsigned ops;
  int es, vbytes;
  int64_t lo, hi;
  int from_wpr, from_iters, wpr, iters;
};
constexpr ShapeOverride kShapeOverrides[] = {
    // 16-bit forward rows of 129-204 vectors (N = 1032-1632), which the rule
    // gives 2 waves x 2 with more than a quarter of the vectors empty: one
    // wave of 4 (no cross-wave sum, eight rows per workgroup).  RMSNorm
    // 16384 x 1096 16-19 % and 16384 x 1600 7 % faster, LayerNorm 4096 x 1160
    // 4 % faster, 4096 x 1600 5 % slower; 12-25 % faster than 3 x 1 at N =
    // 1280 and 1536 (M = 4096 to 65536, both norms).
    {kFwdOps, 2, 16, 129, 204, 2, 2, 1, 4},
    // 16-bit forward rows of 308-320 vectors (N = 2464-2560), rule 3 x 2: one
    // wave of 5, 5-12 % faster at N = 2560.  (Rows of 257-307 vectors get one
    // wave of 5 from the rule itself; exactly 256 keep 2 x 2, one wave of 4
    // was up to 12 % slower; 321-384 keep 3 x 2, one wave of 8 or 4 x 2
    // measured -3 ... +20 %.)
    {kFwdOps, 2, 16, 308, 320, 3, 2, 1, 5},
    // 16-bit LayerNorm forward rows of 641-896 vectors (N = 5128-7168), rule
    // 6 or 7 waves x 2: 3 x 4 or 4 x 4, half the waves in its two cross-wave
    // sums and a persistent grid from M = 8192 on.  N = 5264, 5896, 6144,
    // 6432, 7000, 7168: 3.3-10.5 % faster at M = 8192 and 16384, -0.8 ...
    // +1.3 % at M = 4096.
    {op_bit(RowOp::kLnFwd), 2, 16, 641, 768, 6, 2, 3, 4},
    {op_bit(RowOp::kLnFwd), 2, 16, 769, 896, 7, 2, 4, 4},
    // 16-bit LayerNorm forward rows of 1025-1279 vectors (N = 8200-10232),
    // rule 5 x 4: 4 x 5, eight-wave workgroups of two rows.  1.4-9.8 %
    // faster at M = 4096 to 16384 (N = 8704, 9056, 9216); at exactly 1280
    // vectors (N = 10240, no lane idle in 5 x 4) -2.8 ... +1.6 %, so it keeps
    // the rule's shape.  RMSNorm's forward measured indifferent (+-1 %).
    {op_bit(RowOp::kLnFwd), 2, 16, 1025, 1279, 5, 4, 4, 5},
    // backward rows the rule gives one wave of five vectors (257-320
    // vectors): 3 x 2, fewer row groups per workgroup to add up at its end.
    // fp32 RMSNorm N = 1028-1280: 8.6-14 % faster at M = 4096 to 16384.
    {kBwdOps, 0, 0, 257, 320, 1, 5, 3, 2},
};

// The launch plan of row operation `op` over M rows of N elements of type
// `dtype`, read in vectors of `vec` elements.
// Workgroups of about kBlockWaves waves (rpb = kBlockWaves / wpr row groups
// of wpr waves each), and how many of them fit a CU's kBwdResidentWaves.
inline int64_t workgroups_per_cu(const RowPlan& p) {
  int64_t per_cu = 1;
  while (per_cu * 2 * p.wpr * p.rpb <= kBwdResidentWaves) per_cu *= 2;
  return per_cu;
}

// Forward grid: one workgroup per row group, or persistent where a grid of
// the workgroups that fit the CUs fills every CU with
// kBwdResidentWaves waves, or with at least kFwdPersistentMinWaves waves
// whose lanes each carry four 16-byte vectors, and each workgroup then
// takes at least kFwdPersistentMinSteps row groups (its weights stay in
// registers across them).  Measured on MI355X: 2-4 % faster at 16384 x 8192
// and 8192 x 16384, 7-9 % for LayerNorm at 4096 x 8192 and larger; 7-wave
// rows of four vectors (N = 12800-14336 16-bit, fp32 N = 7168) 0.5-3.6 %
// faster for RMSNorm and 5-10 % for LayerNorm, which loads two weight
// vectors per workgroup; for LayerNorm also 6-wave rows of four vectors
// (12 waves per CU, kLnFwdPersistentMinWaves): 0.7-8 % faster at M = 4096
// to 16384, N = 10752-12288 and fp32 N = 6144, where RMSNorm's were -3 ...
// +3 %.  Elsewhere one workgroup per row group is faster: with fewer waves
// per CU or two vectors per lane a persistent grid keeps too few loads in
// flight (5-wave rows at N = 5120, 10 waves per CU: 8-12 % slower; 7-wave
// rows of two vectors at N = 7168: 1-6 % slower), and with 2-4 row groups
// per workgroup (4096 x 4096, LayerNorm at 4096 x 2048) the rows of a
// workgroup queue behind each other (3-15 % slower).
// A few row steps: 16-bit rows of at least kFwdFewStepsMinRowBytes and at
// most kFwdFewStepsMaxWaves waves, where a grid of kFwdFewStepsGrid
// workgroups of one row group each (four per CU, all resident at once) gives
// every workgroup 3 to 6 row steps (LayerNorm; 3 to 4 for RMSNorm), run as
// that persistent grid: every CU gets the same rows, where the dispatcher's
// rounds of one-row-group workgroups leave the last round part empty, and
// each workgroup loads the weights once.  Measured on MI355X (interleaved
// comparison, fp16 LayerNorm): M = 3000 to 6144, N = 3584-7168 3-13 % faster
// (the chapter's M = 4096 sweep: N = 3584 7 %, 4096 9 %, 4608 9 %, 5120
// 10 %, 5632 13 %, 6144 12 %, 6656 10 %, 7168 9 %, 8704-10240 6-8 %);
// 3072 (6 KiB rows) -4 ... +1 %; rows of 6-7 waves of four vectors, which
// the rules above run persistent with two workgroups per CU, 3-14 % slower
// (N = 10752-14336: four of their workgroups do not all fit a CU); at
// M = 8192 -7 ... +4 % and M = 16384 -7 ... +8 %, M = 2048 -15 ... +19 %,
// M = 1024 -4 ... +3 %, so those keep the rules above; RMSNorm bf16 M = 3000
// and 4096, N = 3072-5120 1-8 % faster (the 4096 x 4096 workload 1 %),
// M = 5000 and 6144 0-1 % slower.
// Shorter 16-bit rows (more than kFwdFewStepsShortMinRowBytes, less than
// kFwdFewStepsMinRowBytes; 16-byte vectors): where the rows divide evenly into
// 2 to 6 row steps (LayerNorm; 2 to 4 for RMSNorm) of workgroups of up to
// kFwdFewStepsShortGroups row groups (kBlockWaves waves at most), on a
// whole number of workgroups per CU (at most four), so that every CU and
// every workgroup takes the same rows, the forward runs as that persistent
// grid.  Measured on MI355X (interleaved comparison against the rules
// below): LayerNorm fp16 N = 2576-3456 (rows of 3-4 waves, two per
// workgroup) at M = 3072, 4096, 6144, 8192, 12288: -1 ... -13 % (the
// chapter's M = 4096 sweep at N = 3072: 11 %), N = 1280-2560 (rows of 1-2
// waves, four per workgroup) at M = 6144-16384: -4 ... -18 % (2048: -4 ...
// +1 % at 3-4 steps); RMSNorm bf16 -1 ... -10 % in the same places.  Where
// the rows do not divide evenly (M = 2100, 2500, 5000, 10000, 14000) the
// same grids, balanced or of four workgroups per CU, ran up to 27 % slower:
// a static grid then leaves some CUs more rows, where the dispatcher
// balances one-step workgroups.  Rows of at most 2 KiB (one or two vectors
// per lane in one wave) were -9 ... +11 %.
constexpr int64_t kFwdFewStepsGrid = 4 * kComputeUnits;
constexpr int64_t kFwdFewStepsMin = 3;
constexpr int64_t kFwdFewStepsMaxLn = 6;
constexpr int64_t kFwdFewStepsMaxRms = 4;
constexpr int64_t kFwdFewStepsMinRowBytes = 7168;
constexpr int kFwdFewStepsMaxWaves = 5;
constexpr int kFwdFewStepsShortGroups = 4;
constexpr int64_t kFwdFewStepsShortMinRowBytes = 2048;
constexpr int64_t kFwdFewStepsShortMin = 2;
inline void plan_fwd_grid(RowPlan& p, RowOp op, int64_t M, int64_t N, int es) {
  const int64_t max_steps = op == RowOp::kLnFwd ? kFwdFewStepsMaxLn : kFwdFewStepsMaxRms;
  const int64_t few_steps = ceil_div(M, kFwdFewStepsGrid);
  if (es == 2 && N * es >= kFwdFewStepsMinRowBytes && p.wpr <= kFwdFewStepsMaxWaves && few_steps >= kFwdFewStepsMin &&
      few_steps <= max_steps) {
    p.rpb = 1;
    p.grid = kFwdFewStepsGrid;
    p.row_iters = few_steps;
    return;
  }
  if (es == 2 && p.vec * es == 16 && N * es > kFwdFewStepsShortMinRowBytes && N * es < kFwdFewStepsMinRowBytes) {
    // One workgroup per CU covers cu_step_rows rows per row step; M holds
    // `units` such blocks of rows (whole ones only), dealt out as `steps` row
    // steps to units / steps workgroups per CU (at most four).
    const int rpb = std::max(1, std::min(kFwdFewStepsShortGroups, kBlockWaves / p.wpr));
    const int64_t cu_step_rows = int64_t(rpb) * kComputeUnits;
    const int64_t units = M / cu_step_rows;
    const int64_t steps = ceil_div(units, kFwdFewStepsGrid / kComputeUnits);
    if (M % cu_step_rows == 0 && steps >= kFwdFewStepsShortMin && steps <= max_steps && units % steps == 0) {
      p.rpb = rpb;
      p.row_iters = steps;
      p.grid = units / steps * kComputeUnits;
      return;
    }
  }
  p.rpb = std::max(1, kBlockWaves / p.wpr);
  const int64_t groups = ceil_div(M, p.rpb);
  const int64_t per_cu = workgroups_per_cu(p);
  const int64_t cu_waves = per_cu * p.wpr * p.rpb;
  const bool four_full_vectors = p.iters == 4 && p.vec * es == 16;
  const bool persistent =
      (cu_waves == kBwdResidentWaves ||
       (cu_waves >= (op == RowOp::kLnFwd ? kLnFwdPersistentMinWaves : kFwdPersistentMinWaves) && four_full_vectors)) &&
      groups >= kFwdPersistentMinSteps * kComputeUnits * per_cu;
  p.grid = std::max<int64_t>(1, std::min(groups, persistent ? kComputeUnits * per_cu : kFwdGridMax));
  p.row_iters = ceil_div(groups, p.grid);
}

// Backward workgroup shape and grid (the backward is always persistent: each
// workgroup loops over its rows and writes one partial row per weight), in
// this order:
//   1. workgroups of about kBlockWaves waves, as many per CU as fit
//      kBwdResidentWaves, at most kBwdGridMax of them;
//   2. where the pipelined row loop is compiled for the plan: one workgroup
//      per CU; where the partial rows of the grid of step 1 exceed
//      kBwdWideShare of the row traffic, rows of 5-8 waves two to a 16-wave
//      workgroup (bwd_partials_heavy);
//   3. where only the narrow build pipelines (bf16 LayerNorm): one workgroup
//      per CU for rows of 1-4 waves, and of 8 waves below
//      kBwdWideShareUnpipelined;
//   4. where the pipelined loop is not compiled: rows of 4-8 waves as one
//      16-wave workgroup per CU, above kBwdWideShareUnpipelined only;
//   5. with one workgroup per CU: at least kBwdMinSteps row steps each while
//      the grid keeps kBwdMinGridWaves waves, then the fewest workgroups that
//      keep the step count and those waves.
// Pipelining (bwd_pipelined) and the partial rows' store policy
// (partials_nontemporal) follow from the resulting plan.
inline void plan_bwd_grid(RowPlan& p, RowOp op, int64_t M, int es, int dtype) {
  p.rpb = std::max(1, kBlockWaves / p.wpr);
  int64_t groups = ceil_div(M, p.rpb);
  int64_t per_cu = workgroups_per_cu(p);
  const int64_t default_grid = std::min(groups, std::min(kBwdGridMax, kComputeUnits * per_cu));
  const bool fits = bwd_pipeline_fits(op, dtype, p.vec, p.iters);
  const bool fits_narrow = bwd_pipeline_fits(op, dtype, p.vec, p.iters, kNarrowThreads) && p.threads() <= kNarrowThreads;
  const bool rows_4_to_8 = p.wpr * 2 >= kBlockWaves && p.wpr <= kBlockWaves;
  const bool rows_5_to_8 = p.wpr * 2 > kBlockWaves && p.wpr <= kBlockWaves;
  const bool heavy_unpipelined = bwd_partials_heavy(op, M, es, default_grid, kBwdWideShareUnpipelined);
  bool sixteen_waves = false;
  if (fits) {
    sixteen_waves = rows_5_to_8 && bwd_partials_heavy(op, M, es, default_grid);
    per_cu = 1;
  } else if (fits_narrow && (p.wpr <= kBlockWaves / 2 || (p.wpr == kBlockWaves && !heavy_unpipelined))) {
    per_cu = 1;  // the bf16 LayerNorm backward, pipelined in its narrow build
  } else if (rows_4_to_8 && heavy_unpipelined) {
    sixteen_waves = true;
    per_cu = 1;
  }
  if (sixteen_waves) {
    p.rpb = std::max(1, static_cast<int>(kBwdResidentWaves) / p.wpr);
    groups = ceil_div(M, p.rpb);
  }
  p.grid = std::max<int64_t>(1, std::min(groups, std::min(kBwdGridMax, kComputeUnits * per_cu)));
  const bool one_per_cu = p.grid <= kComputeUnits;
  const int64_t floor_grid = ceil_div(kBwdMinGridWaves, static_cast<int64_t>(p.wpr) * p.rpb);
  if (one_per_cu) p.grid = std::max<int64_t>(1, std::min(p.grid, std::max(ceil_div(groups, kBwdMinSteps), floor_grid)));
  p.row_iters = ceil_div(groups, p.grid);
  if (one_per_cu) p.grid = std::max<int64_t>(1, std::min(p.grid, std::max(ceil_div(groups, p.row_iters), floor_grid)));
}

inline RowPlan plan_rows(RowOp op, int64_t M, int64_t N, int vec, int dtype) {
  const int es = elsize(dtype);
  RowPlan p{};
  p.vec = vec;
  const bool backward = op == RowOp::kRmsBwd || op == RowOp::kLnBwd;
  const int64_t nvec = N / vec;
  const int cap = std::min(kItersMax, std::max(1, lane_elems_cap(op, es) / vec));
  // The forward prefers rows of at most kFwdRowWaves waves, with more vectors
  // per lane beyond that (measured at N = 16384 bf16: 8 waves x 4 vectors ran
  // 4 % faster than 16 x 2); the backward keeps kLaneVectors.
  const int target =
      backward ? kLaneVectors : static_cast<int>(std::max<int64_t>(kLaneVectors, ceil_div(nvec, int64_t(kWave) * kFwdRowWaves)));
  if (!row_shape(nvec, cap, target, es == 2, backward, &p.wpr, &p.iters)) {
    p.iters = 0;  // cannot happen for N <= RMSNORM_N_MAX
    return p;
  }
  // Shapes measured faster than the rule's choice (the table below).
  for (const ShapeOverride& o : kShapeOverrides) {
    if ((o.ops & op_bit(op)) && (o.es == 0 || o.es == es) && (o.vbytes == 0 || o.vbytes == vec * es) &&
        nvec >= o.lo && nvec <= o.hi && p.wpr == o.from_wpr && p.iters == o.from_iters) {
      p.wpr = o.wpr;
      p.iters = o.iters;
      break;
    }
  }
  if (backward)
    plan_bwd_grid(p, op, M, es, dtype);
  else
    plan_fwd_grid(p, op, M, N, es);
  return p;
}

static_assert(kLnWideHeldChunksMin == (RMSNORM_N_MAX + 1 + 8191) / 8192 && kLnWideHeldChunksMax * 8192 == kLnWideMaxN,
              "the held-row wide backward covers every 16-byte-vector wide row");

inline int64_t partial_rows_bound(int64_t M) { return std::min(M, kBwdGridMax); }
inline int64_t wide_partial_rows_bound(int64_t M) { return std::min(M, kComputeUnits); }

// Plan of the wide LayerNorm kernels, for 16-bit rows beyond RMSNORM_N_MAX
// (up to kLnWideMaxN elements): one 1024-thread workgroup per
// row, iters = chunks of 1024 vectors per row; the backward is persistent,
// one workgroup per CU (each writes one dw and one db partial row), the
// forward takes a row per workgroup.
inline RowPlan plan_ln_wide(bool backward, int64_t M, int64_t N, int vec) {
  RowPlan p{};
  p.wide = true;
  p.vec = vec;
  p.wpr = kMaxBlockWaves;
  p.rpb = 1;
  p.iters = static_cast<int>(ceil_div(N / vec, int64_t(kMaxBlockWaves) * kWave));
  p.grid = std::max<int64_t>(1, std::min(M, backward ? wide_partial_rows_bound(M) : kFwdGridMax));
  p.row_iters = ceil_div(M, p.grid);
  return p;
}

// LayerNorm forward of a 16-bit row beyond RMSNORM_N_MAX: the register plan
// where one exists and its rows span at most kLnWideRegWaves waves (16-byte
// vectors) or kLnWideRegWavesNarrow (narrower vectors, which the wide kernel
// reads twice), else the wide kernel.  Measured on MI355X (interleaved
// comparison, fp16 4096 x N): 16-byte vectors N = 16392 (7 waves) 26 %,
// 18432 19.5 %, 20480 (8 waves) 18 % faster in the register plan, N = 21504
// and 23040 (9 waves) 13-17 %, 23552-32768 (10-13 waves) 22-33 % slower;
// 2- and 4-element vectors N = 16386-16390 (9 waves) 16-21 %, 20482 and
// 20484 (11 waves) 5-12 % faster.
constexpr int kLnWideRegWaves = 8;
constexpr int kLnWideRegWavesNarrow = 11;
inline RowPlan plan_ln_fwd(int64_t M, int64_t N, int vec, int dtype) {
  const RowPlan reg = plan_rows(RowOp::kLnFwd, M, N, vec, dtype);
  if (N <= RMSNORM_N_MAX) return reg;
  const int max_waves = vec * elsize(dtype) == 16 ? kLnWideRegWaves : kLnWideRegWavesNarrow;
  return reg.iters > 0 && reg.wpr <= max_waves ? reg : plan_ln_wide(false, M, N, vec);
}

// Whether the RMSNorm forward issues a workgroup's first row's loads before
// it unpacks the weight, so that the unpacking waits for the weight alone
// (otherwise the row's loads wait for a whole memory round trip at the start
// of every workgroup): for persistent plans and for grids of at most
// kFwdFirstRowEarlyMaxGrid workgroups.  Measured on MI355X (interleaved
// comparison against the plain order): bf16 and fp32, N = 1024-8192 at
// M = 4096-16384, 0.2-11 % faster (4096 x 2048 5-12 %, 4096 x 3072 11 %, the
// headline 0.1-0.3 %); grids of 16384-65536 one-step workgroups (rows of
// 5-7 waves at M >= 16384) were 1.3-4 % slower, with many rounds of
// workgroups resident per CU the start of each one is covered anyway.
constexpr int64_t kFwdFirstRowEarlyMaxGrid = 8 * kComputeUnits;
inline bool fwd_first_row_early(const RowPlan& p) { return p.row_iters > 1 || p.grid <= kFwdFirstRowEarlyMaxGrid; }

// Whether a backward workgroup should keep the next row's loads in flight
// while it works on a row: only where it is alone on its CU (it fills the
// CU's resident waves, or the grid has one workgroup per CU), so no other
// workgroup's loads cover the row's reduction and barrier.  Measured on
// MI355X (bf16): 8192 x 16384, 8192 x 15872, 16384 x 15360 and 16384 x 9216
// row passes 5-9 % faster pipelined; one 8-wave workgroup per CU at LayerNorm
// fp16 4096 x 2048 16 % faster pipelined than not; with two workgroups per
// CU (16384 x 8192, 32768 x 5120) pipelining was 2-8 % slower.  (The planner
// gives two workgroups per CU only where the pipelined loop is not compiled.)
inline bool bwd_pipelined(RowOp op, const RowPlan& p, int dtype) {
  const bool alone_on_cu = p.wpr * p.rpb * 2 > kBwdResidentWaves || p.grid <= kComputeUnits;
  return alone_on_cu && bwd_pipeline_fits(op, dtype, p.vec, p.iters, p.threads());
}

// Whether the backward writes its partial rows (tables x grid x N fp32)
// with the nontemporal policy: where they are kPartialsNtBytes or more, so
// they do not take the place of the rows' own data in the caches, above all
// the 256 MB Infinity Cache, which at M = 4096 holds most of a LayerNorm
// backward's x, dy and dx.  Measured on MI355X (interleaved comparison, full
// backward): LayerNorm fp16 4096 x 4096 (8 MiB of partials) 6.3 %, 4096 x
// 8192 5.3 %, 1151 x 8192 6.5 %, RMSNorm bf16 2048 x 8192 4.6 %, 4096 x 4096
// (4 MiB) 1.6 % faster, 16384 x 8192 and 8192 x 16384 within 0.4 %; at
// LayerNorm 4096 x 1024 (2 MiB), which the column sum reads back from the
// caches, 4.2 % slower, and in the wide LayerNorm kernels (4096 x 24576 and
// 4096 x 32768, 48-64 MiB) 3.5 % slower, so those keep the default policy.
constexpr int64_t kPartialsNtBytes = int64_t(4) << 20;
inline bool partials_nontemporal(int tables, int64_t grid, int64_t N) {
  return static_cast<int64_t>(tables) * grid * N * 4 >= kPartialsNtBytes;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? RMSNORM_OK : RMSNORM_E_HIP; }

}  // namespace rmsn
