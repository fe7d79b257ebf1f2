// Internal launch interface between the C ABI (abi.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <type_traits>
#include <utility>

namespace adaln {

// Error reporting of the C ABI: fail() records a message for
// adaln_last_error() and returns `code`; ok() clears it.
int fail(int code, const char *fmt, ...);
int ok();

// How a token row is spread over a workgroup: W wavefronts share one row and
// each lane holds V 16-byte vectors of it (vector k of wave w, lane l is the
// row's vector (k*W + w)*64 + l).  A 256-thread workgroup works on 4/W rows.
//
// ADALN_ROW_PLANS lists the instantiated (V, W) pairs, smallest W first and,
// within one W, smallest V first; the planner takes the first that holds the
// row.  The largest row is 16 * 4 * 64 = 4096 vectors.
#define ADALN_ROW_PLANS(X)                                                   \
  X(1, 1) X(2, 1) X(3, 1) X(4, 1) X(5, 1) X(6, 1) X(8, 1) X(10, 1) X(12, 1) \
  X(16, 1) X(12, 2) X(16, 2) X(12, 4) X(16, 4)

struct RowPlan {
  int V = 0;
  int W = 0;
};

// The D-tile reduction grid: (d_tiles, n_tiles, B) workgroups, each covering
// 64 vectors of features (one per lane) and n_tile token rows of one sample.
struct DmodPlan {
  int d_tiles = 0;
  int n_tile = 0;
  int n_tiles = 0;
};

// Row-stream kernels (the forward and the fused backward): W wavefronts per
// row, lane l of wavefront h holding vectors (h*V + k)*64 + l, k < V.  A
// persistent grid of `grid` four-wavefront workgroups: the samples are
// processed `groups` at a time, with `bps` workgroups per sample, and each
// row walker (one wavefront, or the W of a row) walks its sample's rows with
// a stride of (4/W)*bps.  The forward instead covers the rows with its grid
// (bps = groups = 0, `grid` workgroups of 4/W rows).
struct StreamPlan {
  int V = 0;       // vectors per lane
  int W = 1;       // wavefronts per row (2, 4 or 8: rows too wide for one)
  int64_t grid = 0;
  int bps = 0;     // workgroups per sample (partial rows per sample)
  int groups = 0;  // samples in flight
  int skew = 0;    // sample b's walk starts (b * skew) % N rows in
};

// How a stream kernel's workgroups map to token rows.  UniformMap: B samples
// of N rows, `groups` samples in flight, bps workgroups per sample; a
// workgroup visits samples slot, slot + groups, ...  SegMap: up to
// kMaxSegments segments of any length, segment s owning the workgroups
// [wg_start[s], wg_start[s+1]) and the rows [row_start[s], row_start[s+1]),
// modulated by vector mod[s].  Either way each (segment, workgroup) pair
// writes one partial row: row part_row of the backward's workspace.
struct UniformMap {
  int32_t B;
  int32_t N;
  int32_t bps;
  int32_t groups;
  int32_t skew;  // sample b's walk starts (b * skew) % N rows in
};

constexpr int kMaxSegments = 128;

struct SegMap {
  int32_t nseg;
  int32_t wg_start[kMaxSegments + 1];
  int32_t mod[kMaxSegments];
  int64_t row_start[kMaxSegments + 1];
};

// Token row -> modulation vector, for the forward's grids over the rows.
// BatchRows: B samples of N rows (row r belongs to sample r / N; B * N <=
// 2^31 - 1).  SegMap: the segment s with row_start[s] <= r < row_start[s+1]
// (the last s with row_start[s] <= r skips the empty segments before it).
struct BatchRows {
  int32_t N;
};

__device__ __forceinline__ int row_mod(const BatchRows &m, int64_t r) {
  return (int)((uint32_t)r / (uint32_t)m.N);
}

__device__ __forceinline__ int row_mod(const SegMap &m, int64_t r) {
  int lo = 0, hi = m.nseg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (m.row_start[mid] <= r)
      lo = mid;
    else
      hi = mid - 1;
  }
  return m.mod[lo];
}

// Calls f(row0, rows, mod, k_in, bps, part_row, rot) for each segment the
// calling workgroup works on; a kernel visits the segment's rows in the
// order n = 0, 1, ..., rows - 1 of its walk, at row row0 + (n + rot) mod
// rows.  Workgroup-uniform, so a kernel may place barriers in f.
template <class F>
__device__ __forceinline__ void for_each_segment(const UniformMap &m, F &&f) {
  const int slot = blockIdx.x / m.bps;
  const int k_in = blockIdx.x - slot * m.bps;
  if (slot >= m.groups) return;
  for (int b = slot; b < m.B; b += m.groups)
    f((int64_t)b * m.N, m.N, b, k_in, m.bps, b * m.bps + k_in,
      m.skew > 0 && m.N > 0 ? (int)(((int64_t)b * m.skew) % m.N) : 0);
}

template <class F>
__device__ __forceinline__ void for_each_segment(const SegMap &m, F &&f) {
  const int bid = blockIdx.x;
  if (bid >= m.wg_start[m.nseg]) return;
  int lo = 0, hi = m.nseg - 1;  // last s with wg_start[s] <= bid
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (m.wg_start[mid] <= bid)
      lo = mid;
    else
      hi = mid - 1;
  }
  // segments without rows own no workgroups, so wg_start[lo + 1] > bid
  const int s = lo;
  const int bps = m.wg_start[s + 1] - m.wg_start[s];
  f(m.row_start[s], (int)(m.row_start[s + 1] - m.row_start[s]), m.mod[s],
    bid - m.wg_start[s], bps, bid, 0);
}

#define ADALN_STREAM_V(X) X(1) X(2) X(3) X(4) X(5) X(6) X(8) X(10) X(12) X(16)
#define ADALN_BWD_STREAM_V(X) X(1) X(2) X(3) X(4) X(5)
constexpr int kMaxStreamVectors = 16 * 64;

// Rows in flight per wavefront (PF) and waves per SIMD (OCC) of each
// persistent stream kernel instantiation.  OCC also fixes the grid: OCC
// workgroups per CU.
// Short rows get two rows in flight and several workgroups per CU to keep
// enough bytes in flight; long rows get the whole register file of one
// wavefront per SIMD (the backward's per-lane accumulators need it).  The
// ADALN_* macros in this part only override the measured choices at build
// time, to measure the alternatives; the library is built without them.
#ifndef ADALN_BWD_PF_SHORT
#define ADALN_BWD_PF_SHORT 2
#endif
#ifndef ADALN_BWD_PF_LONG
#define ADALN_BWD_PF_LONG 1
#endif
#ifndef ADALN_BWD_OCC_SHORT
#define ADALN_BWD_OCC_SHORT 2
#endif
#ifndef ADALN_BWD_OCC_LONG
#define ADALN_BWD_OCC_LONG 1
#endif
#ifndef ADALN_BWD_SHORT_V
#define ADALN_BWD_SHORT_V 3
#endif
// End of a sample in bwd_stream_kernel: where the four wavefronts'
// accumulators fit 48 KiB of LDS together (bf16 rows of up to 3 vectors per
// lane, f32 up to 5), all four stage them at once and each adds and writes a
// quarter of the partial row (one barrier); wider rows stage them one
// wavefront at a time into wavefront 0.  The sums run in wavefront order
// either way.  Measured on MI355X (fused backward + finish, paired, same
// buffers): bf16 16 x 1560 x 1536 48.6 -> 47.5 us, 64 x 1024 x 768 63.8 ->
// 63.0 us, one sample within noise.
constexpr bool bwd_stage_all(int V, int E) {
  return 4 * V * E * 2 * 64 * 4 <= 48 * 1024;
}
constexpr int bwd_stream_pf(int V) {
  return V <= 6 ? ADALN_BWD_PF_SHORT : ADALN_BWD_PF_LONG;
}
constexpr int bwd_stream_occ(int V) {
  return V <= ADALN_BWD_SHORT_V ? ADALN_BWD_OCC_SHORT : ADALN_BWD_OCC_LONG;
}
// The fused backward keeps per-lane accumulators (2*V*E floats) next to the
// row.  One wavefront per row (bwd_stream_kernel) holds rows of up to 320
// vectors.  Wider rows split between the W wavefronts of a row group
// (bwd_wide_kernel), V vectors per lane each: pairs up to 2 * 640 vectors,
// quads (W = 4) up to 4 * 640; past 2560 vectors the accumulators outgrow
// the register file of a four-wavefront workgroup, and eight wavefronts (a
// 512-thread workgroup, two per SIMD) share the row, up to 8 * 512 vectors,
// the widest row of the library.  A whole 640-vector row in one wavefront needs
// the full register file at one wavefront per SIMD, so nothing covers its
// memory latency while it computes; as halves, rows of up to 640 vectors run
// at two wavefronts per SIMD (measured on MI355X: the D = 5120 bf16 backward
// 411 -> 400 us, D = 3072 1-3% faster).
constexpr int kMaxBwdStreamV = 5;
#define ADALN_BWD_PAIR_V(X) X(3) X(4) X(5) X(6) X(8) X(10)
#define ADALN_BWD_QUAD_V(X) X(6) X(8) X(10)
#define ADALN_BWD_OCT_V(X) X(6) X(8)
// Threads per workgroup of bwd_wide_kernel: four wavefronts, or eight for
// rows split eight ways.
constexpr int bwd_wide_block(int W) { return W == 8 ? 512 : 256; }
// Waves per SIMD of bwd_wide_kernel (an eight-wavefront workgroup puts two on
// each SIMD), and so workgroups per CU: occ * 4 * 64 / threads.
constexpr int bwd_wide_occ(int V, int W) {
  return W == 8 || V <= 5 ? 2 : 1;
}
constexpr int bwd_wide_wgs_per_cu(int V, int W) {
  return bwd_wide_occ(V, W) * 4 * 64 / bwd_wide_block(W);
}
// Rows in flight per wavefront of bwd_wide_kernel (E elements per vector):
// bf16 rows at one wavefront per SIMD take a second row where its 2*V
// vectors of x and dy fit beside the accumulators without spills (V*E <= 64
// elements; <= 48 where the row ends inside a wavefront's vectors and the
// tail needs registers of its own).  Measured on MI355X (fused backward,
// bf16): D = 6144 288 -> 262 us, D = 8192 471 -> 440 us, D = 12288 555 ->
// 517 us, D = 16384 586 -> 540 us.  f32 rows gained at most 2% and keep one.
constexpr int bwd_wide_pf(int V, int W, int E, bool full) {
#ifdef ADALN_BWD_WIDE_PF1
  return 1;
#else
  return bwd_wide_occ(V, W) == 1 && E == 8 && V * E <= (full ? 64 : 48) ? 2
                                                                         : 1;
#endif
}
// Registers of bf16 rows split eight ways: two wavefronts per SIMD leave 256
// registers each, and at 8 vectors per lane the accumulators (128), the row
// (64) and the scale (32) spill.  There bwd_wide_kernel reads the scale
// again (from L2) at each use instead of holding it for the whole segment,
// and, from 6 vectors per lane, derives its vector indices again in each row
// instead of holding them (no spills left; bf16 1 x 12000 x 32768: 1768 us
// with 398 spilled registers, 513 us without).
constexpr bool bwd_wide_scale_regs(int V, int W, int E) {
  return !(W == 8 && E == 8 && V >= 8);
}
constexpr bool bwd_wide_index_regs(int V, int W, int E) {
  return !(W == 8 && E == 8);
}
// XCD-weighted walk of bwd_wide_kernel.  Its workgroups each take a fixed
// share of a sample's rows, and the kernel ends with its slowest workgroup.
// A copy of the kernel that records each wavefront's clock showed the
// workgroups on odd XCDs (odd block index: workgroups go to the eight XCDs
// in turn) finishing their rows about 4% after those on even XCDs, run after
// run, for bf16 rows split between a pair of wavefronts at two wavefronts per
// SIMD.  There, after every m rounds of the walk, the walkers of even-XCD
// workgroups take one extra row each, so that all XCDs finish together
// (every row still visited once; the partial sums change grouping, not
// precision).  Measured on MI355X (backward + finish, HIP events, same
// buffers, two boxes): 1 x 75600 x 5120 401-404 -> 386-388 us (m = 16),
// 3 x 20000 x 5120 333.5 -> 321.5 us; D = 3072 (m = 12) 84 x 1560 459-462 ->
// 443-446 us, 16 x 8190 429-433 -> 421-426 us, 32 x 1560 179.8 -> 177.5 us.
// Rows of 4 vectors per lane were unchanged, and ragged rows, f32 rows,
// quads and rows at one wavefront per SIMD 2-5% slower: those keep m = 0,
// the plain walk, and so do the packed layouts (the two-stream pack 1%
// slower with it, the mixed pack unchanged).
constexpr int bwd_wide_xcd_m(int V, int W, int E, bool full) {
  return E == 8 && W == 2 && full ? (V == 5 ? 16 : V == 3 ? 12 : 0) : 0;
}
// Loop form of bwd_wide_kernel at one row in flight: the loads as one step
// and the arithmetic as the next, or both in one branch.  The compiler
// schedules the two forms differently, and on MI355X neither wins
// everywhere (fused backward, HIP events): the split form for f32 rows and
// rows of up to 4 vectors per lane (bf16 84 x 1560 x 3072 463 -> 397-454 us,
// 4 x 30000 x 2568 446 -> 387-399 us, f32 1 x 120000 x 1288 411 -> 334-348
// us), one branch for bf16 rows of 5 and 10 (1 x 75600 x 5120 410-415 ->
// 403-405 us, 1 x 24000 x 20480 604 -> 587-591 us).
constexpr bool bwd_wide_split(int V, int E) {
#if defined(ADALN_BWD_WIDE_SPLIT_ALL)
  return true;
#elif defined(ADALN_BWD_WIDE_SPLIT_NONE)
  return false;
#else
  return E == 4 || V <= 4;
#endif
}

// The forward kernels (fwd_rows_kernel, fwd_wide_kernel) widen x again for
// the variance pass and x, scale and shift again for the output where keeping
// them widened would leave one wavefront per SIMD: bf16 rows of 16 vectors
// per lane (256 -> 216-252 VGPRs, two wavefronts per SIMD).  Measured on
// MI355X, bf16, D = 8192: 16 x 1560 rows 160.4 -> 143.1 us, 1 x 16384 106.5
// -> 96.6 us; at 10 vectors per lane (two -> three wavefronts per SIMD) it
// costs 5% (1 x 75600 x 5120 256.4 -> 268.1 us), and 6 vectors 3%.
constexpr bool fwd_rows_rewiden(int V, int E) { return E == 8 && V >= 16; }
// fwd_wide_kernel loads scale and shift after the row's statistics, vector
// by vector in the output pass (an empty asm statement keeps the loads
// there), for f32 rows of 16 vectors per lane that end inside a wavefront's
// vectors: 225-236 -> 129-134 VGPRs, three wavefronts per SIMD instead of
// two.  Measured on MI355X (forward, HIP events, same buffers): f32
// 1 x 16384 x 12292 323 -> 303 us, 1 x 30000 x 14000 647 -> 608 us; rows
// that fill all 16 vectors were 8-12% slower that way and keep the early
// loads.
constexpr bool fwd_wide_late_mod(int V, int E, bool full) {
  return E == 4 && V >= 16 && !full;
}

// The forward of rows wider than 1024 vectors splits each row between the W
// wavefronts of a row group (fwd_wide_kernel), V vectors per lane each:
// pairs up to 1536 vectors, quads up to 4096.
#define ADALN_FWD_PAIR_V(X) X(10) X(12)
#define ADALN_FWD_QUAD_V(X) X(8) X(10) X(12) X(16)

constexpr int kCUs = 256;  // compute units of an MI355X

// Grid-stride kernels take at most this many workgroups per launch.
constexpr int64_t kMaxGrid = 1 << 20;

// Launch `k` with min(blocks, kMaxGrid) workgroups of 256 threads; returns the
// launch's own status (no global error state involved).
template <typename... P, typename... A>
inline hipError_t launch_kernel(void (*k)(P...), int64_t blocks,
                                hipStream_t s, A... args) {
  static_assert(std::is_same<std::tuple<P...>, std::tuple<A...>>::value,
                "kernel arguments must match the kernel's parameter types");
  if (blocks <= 0) return hipSuccess;
  const unsigned grid = (unsigned)(blocks < kMaxGrid ? blocks : kMaxGrid);
  void *argv[] = {(void *)&args...};
  return hipLaunchKernel((const void *)k, dim3(grid), dim3(256), argv, 0, s);
}

// As launch_kernel, with `threads` threads and `lds` bytes of dynamic LDS
// per workgroup.
template <typename... P, typename... A>
inline hipError_t launch_kernel_lds(void (*k)(P...), int64_t blocks,
                                    int threads, size_t lds, hipStream_t s,
                                    A... args) {
  static_assert(std::is_same<std::tuple<P...>, std::tuple<A...>>::value,
                "kernel arguments must match the kernel's parameter types");
  if (blocks <= 0) return hipSuccess;
  const unsigned grid = (unsigned)(blocks < kMaxGrid ? blocks : kMaxGrid);
  void *argv[] = {(void *)&args...};
  return hipLaunchKernel((const void *)k, dim3(grid), dim3(threads), argv, lds,
                         s);
}

// As launch_kernel, with `threads` threads per workgroup.
template <typename... P, typename... A>
inline hipError_t launch_kernel_threads(void (*k)(P...), int64_t blocks,
                                        int threads, hipStream_t s,
                                        A... args) {
  static_assert(std::is_same<std::tuple<P...>, std::tuple<A...>>::value,
                "kernel arguments must match the kernel's parameter types");
  if (blocks <= 0) return hipSuccess;
  const unsigned grid = (unsigned)(blocks < kMaxGrid ? blocks : kMaxGrid);
  void *argv[] = {(void *)&args...};
  return hipLaunchKernel((const void *)k, dim3(grid), dim3(threads), argv, 0,
                         s);
}

// Returns false if no instantiation holds a row of nvec vectors.
bool choose_row_plan(int64_t nvec, RowPlan *plan);
int64_t max_row_vectors();

DmodPlan choose_dmod_plan(int64_t B, int64_t N, int64_t nvec);
// Row-stream plan for the forward (bwd = false) or the fused backward; false
// when the row is wider than kMaxStreamVectors.
bool choose_stream_plan(int64_t B, int64_t N, int64_t nvec, bool bwd,
                        StreamPlan *plan);

// Launchers: enqueue on `stream` and return the launch's own status.
hipError_t launch_bwd_dx(int dtype, const RowPlan &plan, const void *dy,
                         const void *x, const void *scale, const float *mean,
                         const float *rstd, void *dx, int64_t rows, int32_t N,
                         int32_t D, hipStream_t stream);

// D-tile partial sums only (no finish).
hipError_t launch_dmod_partial(int dtype, const DmodPlan &plan,
                               const void *dy, const void *x,
                               const float *mean, const float *rstd,
                               float *part_scale, float *part_shift,
                               int32_t B, int32_t N, int32_t D,
                               hipStream_t stream);

// Launch shape of the finishing kernels for `vectors` modulation vectors
// (samples) of D features whose largest sum has `rows` partial rows: column
// blocks of F features, wpc wavefronts per block, cpb blocks per workgroup
// of `threads` threads, `blocks` workgroups (the kernel strides over more
// than kMaxGrid).
struct FinishPlan {
  int F = 0;
  int wpc = 0;
  int cpb = 0;
  int threads = 0;
  int32_t col_blocks = 0;
  int64_t total_cols = 0;
  int64_t blocks = 0;
};
FinishPlan finish_plan(int64_t vectors, int32_t D, int64_t rows);

// dscale/dshift = sums over n_tiles of [B, n_tiles, D] partials, in index
// order (zero when n_tiles == 0).
hipError_t launch_dmod_finish(const float *part_scale,
                              const float *part_shift, float *dscale,
                              float *dshift, int32_t B, int32_t D,
                              int32_t n_tiles, hipStream_t stream);

// The forward of one-wavefront rows (V vectors per lane): one launch per
// 2^22 rows, one row per wavefront.
hipError_t launch_fwd_rows(int dtype, int V, const void *x, const void *scale,
                           const void *shift, void *y, float *mean,
                           float *rstd, int32_t B, int32_t N, int32_t D,
                           hipStream_t stream);

hipError_t launch_fwd_wide(int dtype, const StreamPlan &plan, const void *x,
                           const void *scale, const void *shift, void *y,
                           float *mean, float *rstd, int32_t B, int32_t N,
                           int32_t D, hipStream_t stream);

hipError_t launch_fwd_wide_segments(int dtype, const StreamPlan &plan,
                                    const SegMap &map, const void *x,
                                    const void *scale, const void *shift,
                                    void *y, float *mean, float *rstd,
                                    int32_t D, hipStream_t stream);

hipError_t launch_fwd_segments(int dtype, int V, const SegMap &map,
                               const void *x, const void *scale,
                               const void *shift, void *y, float *mean,
                               float *rstd, int32_t D, hipStream_t stream);

hipError_t launch_bwd_wide(int dtype, const StreamPlan &plan, const void *dy,
                           const void *x, const void *scale,
                           const float *mean, const float *rstd, void *dx,
                           float *part_scale, float *part_shift, int32_t B,
                           int32_t N, int32_t D, hipStream_t stream);

hipError_t launch_bwd_wide_segments(int dtype, const StreamPlan &plan,
                                    const SegMap &map, const void *dy,
                                    const void *x, const void *scale,
                                    const float *mean, const float *rstd,
                                    void *dx, float *part_scale,
                                    float *part_shift, int32_t D,
                                    hipStream_t stream);

hipError_t launch_bwd_segments(int dtype, int V, const SegMap &map,
                               const void *dy, const void *x,
                               const void *scale, const float *mean,
                               const float *rstd, void *dx, float *part_scale,
                               float *part_shift, int32_t D,
                               hipStream_t stream);

// dscale[m] / dshift[m] = sum over the segments s with mod[s] == m, in index
// order, of their workgroups' partial rows, in order (zero for an m no
// segment uses).
hipError_t launch_finish_segments(const float *part_scale,
                                  const float *part_shift, float *dscale,
                                  float *dshift, const SegMap &map,
                                  int32_t nmod, int32_t D,
                                  hipStream_t stream);

hipError_t launch_bwd_fused(int dtype, const StreamPlan &plan, const void *dy,
                            const void *x, const void *scale,
                            const float *mean, const float *rstd, void *dx,
                            float *part_scale, float *part_shift, int32_t B,
                            int32_t N, int32_t D, hipStream_t stream);

}  // namespace adaln
