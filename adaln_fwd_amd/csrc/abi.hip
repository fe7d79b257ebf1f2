// C ABI of the fused AdaLN library: argument validation, launch planning and
// dispatch.  Declarations, layouts and error behaviour are documented in
// include/adaln.h.  Every check runs on the host before any HIP call, so an
// invalid call enqueues nothing.
#include <stdarg.h>
#include <algorithm>
#include <mutex>
#include <stdio.h>
#include <stdint.h>

#include "adaln.h"
#include "launch.hpp"

#define ADALN_API extern "C" __attribute__((visibility("default")))

namespace adaln {
namespace {
thread_local char g_msg[256] = "";
}  // namespace

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof g_msg, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_msg[0] = '\0';
  return ADALN_OK;
}

namespace {

int hip_fail(hipError_t e, const char *what) {
  return fail(ADALN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int elems_per_vec(int dtype) { return dtype == ADALN_BF16 ? 8 : 4; }

constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxB = int64_t(1) << 20;

// Checks shared by every operator entry point.
int check_shape(int64_t B, int64_t N, int64_t D, int dtype) {
  if (dtype != ADALN_F32 && dtype != ADALN_BF16)
    return fail(ADALN_ERR_DTYPE, "unknown dtype code %d", dtype);
  if (B < 0 || N < 0)
    return fail(ADALN_ERR_INVALID, "negative size: B=%lld N=%lld",
                (long long)B, (long long)N);
  if (D <= 0)
    return fail(ADALN_ERR_INVALID, "D must be positive, got %lld",
                (long long)D);
  const int E = elems_per_vec(dtype);
  if (D % E != 0)
    return fail(ADALN_ERR_ALIGN, "D=%lld is not a multiple of %d", (long long)D,
                E);
  if (D > adaln_max_d(dtype))
    return fail(ADALN_ERR_UNSUPPORTED, "D=%lld exceeds the largest row (%lld)",
                (long long)D, (long long)adaln_max_d(dtype));
  if (B > kMaxB)
    return fail(ADALN_ERR_INVALID, "B=%lld exceeds %lld", (long long)B,
                (long long)kMaxB);
  if (N > 0 && B > kMaxRows / N)
    return fail(ADALN_ERR_INVALID, "B*N exceeds 2^31-1 rows");
  if (B > kMaxRows / D)
    return fail(ADALN_ERR_INVALID, "B*D exceeds 2^31-1");
  return ADALN_OK;
}

// A pointer is needed when its tensor has elements; it must then be non-NULL
// and 16-byte aligned.
int check_ptr(const void *p, bool needed, const char *name) {
  if (!needed) return ADALN_OK;
  if (p == nullptr) return fail(ADALN_ERR_INVALID, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
    return fail(ADALN_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return ADALN_OK;
}

#define ADALN_TRY(expr)          \
  do {                           \
    const int rc_ = (expr);      \
    if (rc_ != ADALN_OK) return rc_; \
  } while (0)

size_t partial_bytes(int64_t n_tiles, int64_t B, int64_t D) {
  return (size_t)2 * (size_t)B * (size_t)n_tiles * (size_t)D * sizeof(float);
}

// One workspace size serves adaln_bwd (fused plan) and adaln_bwd_dmod
// (D-tile plan).
size_t workspace_bytes(int64_t B, int64_t N, int64_t D, int dtype) {
  const int64_t nvec = D / elems_per_vec(dtype);
  const DmodPlan dp = choose_dmod_plan(B, N, nvec);
  StreamPlan sp;
  const size_t a = partial_bytes(dp.n_tiles, B, D);
  const size_t b = choose_stream_plan(B, N, nvec, true, &sp)
                       ? partial_bytes(sp.bps, B, D)
                       : 0;
  return a > b ? a : b;
}

}  // namespace

// ------------------------------------------------------------------ planning

bool choose_row_plan(int64_t nvec, RowPlan *plan) {
#define ADALN_PLAN_CASE(V_, W_)                 \
  if ((int64_t)(V_) * (W_) * 64 >= nvec) {       \
    plan->V = V_;                               \
    plan->W = W_;                               \
    return true;                                \
  }
  ADALN_ROW_PLANS(ADALN_PLAN_CASE)
#undef ADALN_PLAN_CASE
  return false;
}

int64_t max_row_vectors() {
  int64_t m = 0;
#define ADALN_MAX_CASE(V_, W_) \
  if ((int64_t)(V_) * (W_) * 64 > m) m = (int64_t)(V_) * (W_) * 64;
  ADALN_ROW_PLANS(ADALN_MAX_CASE)
#undef ADALN_MAX_CASE
  return m;
}

// The D-tile grid.  A d_tile is 64 vectors (one per lane of a wavefront).
// n_tile is chosen so the whole grid has about 2048 workgroups (8 per CU on a
// 256-CU part) and is a multiple of 16 rows; it depends only on the shape, so
// the workspace size is a pure function of the arguments.
DmodPlan choose_dmod_plan(int64_t B, int64_t N, int64_t nvec) {
  DmodPlan p;
  p.d_tiles = (int)((nvec + 63) / 64);
  if (B == 0 || N == 0) return p;
  constexpr int64_t kTargetBlocks = 2048;
  const int64_t per_sample_cols = (int64_t)p.d_tiles * B;
  int64_t tiles_per_sample =
      (kTargetBlocks + per_sample_cols - 1) / per_sample_cols;
  if (tiles_per_sample < 1) tiles_per_sample = 1;
  int64_t n_tile = (N + tiles_per_sample - 1) / tiles_per_sample;
  n_tile = (n_tile + 15) / 16 * 16;
  if (n_tile < 16) n_tile = 16;
  p.n_tile = (int)n_tile;
  p.n_tiles = (int)((N + n_tile - 1) / n_tile);
  return p;
}

// Row-stream plans (rows of up to 4096 vectors; the backward takes a pair of
// wavefronts per row past 320 vectors, four past 1280 and eight past 2560;
// the forward a pair past 1024 and four past 1536).  V is the smallest
// instantiated count that holds the row.
//
// The forward covers the rows with its grid, one row per row walker (a
// wavefront, or the W wavefronts sharing a row): ceil(B * N * W / 4)
// workgroups in all (fwd_rows_kernel and fwd_wide_kernel have the
// measurements).
//
// The backward runs a persistent grid: the occupancy OCC fixes G = 256 *
// OCC workgroups (OCC per CU on a 256-CU MI355X), spread over the samples:
// up to G / B workgroups per sample (at least one), `groups` = G / bps
// samples in flight.  Of the counts that keep the most rows any row walker (a
// wavefront, or the W wavefronts sharing a row) visits as low as G / B does,
// bps is the smallest, so that all walkers finish together rather than a few
// walking one row more (measured on MI355X: the 16 x 1560-token, D = 1536
// backward 1% faster).  The plan depends only on the shape, so the workspace
// size ([B, bps, D] partial sums of the backward) is a pure function of it;
// on a part with another CU count the kernels remain correct and only use
// the GPU less evenly.
#ifndef ADALN_BWD_MIN_BPS
#define ADALN_BWD_MIN_BPS 1
#endif

// Backward of one-wavefront rows with many samples: sample b's walk starts
// (b * 97) % N rows into the sample instead of at row 0.  Every sample's
// workgroups sweep their own window of rows; started at the same row, the B
// windows move in step through addresses a fixed multiple of the sample size
// apart, and HBM serves that worse than windows offset from each other.
// Measured on MI355X (fused backward, bf16, D = 1536): 16 x 1560 rows 49.8
// -> 45.2 us, 32 x 780 55.3 -> 45.5 us, 96 x 260 45.7 -> 45.8 us, 2 to 8
// samples within 1% either way; offsets of 13 to 389 rows all helped at 16
// and 32 samples, 97 the most overall.  The pair-of-wavefronts backward
// (wider rows) keeps the aligned start: there the offsets cost 2-4% at
// D = 3072 with 16 and 84 samples.
constexpr int kBwdSkewRows = 97;
constexpr int64_t kBwdSkewMinSamples = 16;

// Samples of at least this many rows count as long for the backward's plan.
constexpr int64_t kLongSample = 4096;

// Waves per SIMD (and so workgroups per CU) the backward's kernel runs at.
// (Workgroups per CU: the same as waves per SIMD for four-wavefront
// workgroups, half of it for the eight-wavefront one.)
int stream_occ(const StreamPlan &p) {
  return p.W > 1 ? bwd_wide_wgs_per_cu(p.V, p.W) : bwd_stream_occ(p.V);
}

// Rows a workgroup works on at a time: 4 / W for the four-wavefront
// workgroups, one for the eight-wavefront backward.
int64_t rows_per_workgroup(int W) { return W >= 4 ? 1 : 4 / W; }

bool choose_stream_plan(int64_t B, int64_t N, int64_t nvec, bool bwd,
                        StreamPlan *plan) {
  StreamPlan p;
#define ADALN_STREAM_PLAN_CASE(V_) \
  if (p.V == 0 && 64 * V_ >= nvec) p.V = V_;
  ADALN_STREAM_V(ADALN_STREAM_PLAN_CASE)
#undef ADALN_STREAM_PLAN_CASE
  if (bwd && (p.V == 0 || p.V > kMaxBwdStreamV)) {
    // too wide for one wavefront's registers: a pair of wavefronts per row,
    // a quad past 1280 vectors, eight past 2560
    p.V = 0;
#define ADALN_PAIR_PLAN_CASE(V_) \
  if (p.V == 0 && (int64_t)2 * 64 * V_ >= nvec) p.V = V_, p.W = 2;
    ADALN_BWD_PAIR_V(ADALN_PAIR_PLAN_CASE)
#undef ADALN_PAIR_PLAN_CASE
#define ADALN_QUAD_PLAN_CASE(V_) \
  if (p.V == 0 && (int64_t)4 * 64 * V_ >= nvec) p.V = V_, p.W = 4;
    ADALN_BWD_QUAD_V(ADALN_QUAD_PLAN_CASE)
#undef ADALN_QUAD_PLAN_CASE
#define ADALN_OCT_PLAN_CASE(V_) \
  if (p.V == 0 && (int64_t)8 * 64 * V_ >= nvec) p.V = V_, p.W = 8;
    ADALN_BWD_OCT_V(ADALN_OCT_PLAN_CASE)
#undef ADALN_OCT_PLAN_CASE
  }
  if (!bwd && p.V == 0) {
    // the forward of rows past 1024 vectors: a pair of wavefronts per row,
    // or a quad past 1536 vectors
#define ADALN_PAIR_PLAN_CASE(V_) \
  if (p.V == 0 && (int64_t)2 * 64 * V_ >= nvec) p.V = V_, p.W = 2;
    ADALN_FWD_PAIR_V(ADALN_PAIR_PLAN_CASE)
#undef ADALN_PAIR_PLAN_CASE
#define ADALN_QUAD_PLAN_CASE(V_) \
  if (p.V == 0 && (int64_t)4 * 64 * V_ >= nvec) p.V = V_, p.W = 4;
    ADALN_FWD_QUAD_V(ADALN_QUAD_PLAN_CASE)
#undef ADALN_QUAD_PLAN_CASE
  }
  if (p.V == 0) return false;
  if (!bwd) {
    const int64_t walkers = rows_per_workgroup(p.W);
    p.grid = (B * N + walkers - 1) / walkers;
  } else if (B > 0 && N > 0) {
    const int occ = stream_occ(p);
    const int64_t G = (int64_t)kCUs * occ;
    const int64_t min_bps = ADALN_BWD_MIN_BPS;
    int64_t bps = G / B > 1 ? G / B : 1;
    const int64_t walkers = rows_per_workgroup(p.W);  // row walkers
    if (B > 1 && N >= kLongSample && p.W > 1) {
      // Long samples: the fewest samples in flight (g, a divisor of B, so
      // every group slot walks B / g samples) that still give each row
      // walker 16 rows of a sample (the backward with pairs or quads of
      // wavefronts per row).  Measured on MI355X, D = 3072, whole backward
      // with pairs of wavefronts per row, although every extra workgroup on
      // a sample costs a partial row: 16 x 8190 443 -> 431 us, 8 x 16380
      // 444 -> 424 us, 4 x 32760 424 -> 422 us.  For samples of 1560 tokens
      // fewer in flight is slower, hence the length threshold; the
      // one-wavefront backward keeps one sample per slot.
      for (int64_t g = 1; g < B && g <= G; ++g) {
        if (B % g == 0 && G / g <= N / (16 * walkers)) {
          bps = G / g;
          break;
        }
      }
    }
    if (bps < min_bps) bps = min_bps < G ? min_bps : G;
    const int64_t most = (N + walkers * bps - 1) / (walkers * bps);
    const int64_t even = (N + walkers * most - 1) / (walkers * most);
    if (even >= min_bps && even < bps) bps = even;
    const int64_t groups = G / bps;
    p.bps = (int)bps;
    p.groups = (int)groups;
    p.grid = (int)(bps * (groups < B ? groups : B));
    if (p.W == 1 && B >= kBwdSkewMinSamples) p.skew = kBwdSkewRows;
  }
  *plan = p;
  return true;
}

// Segment plans.  The G = 256 * OCC workgroups that are resident at once
// (OCC for the kernel's occupancy) are shared out so that the most rows any
// workgroup walks, R, is as small as possible: segment s of N_s rows gets
// ceil(N_s / R) workgroups (none if it is empty), with R the smallest value
// for which the total stays within G -- found by bisection, since the total
// only falls as R grows.  Plain proportional shares (floor(G * N_s / T))
// would leave a short segment, such as the text tokens of a two-stream
// sample, one workgroup with twice the rows of the rest, and the whole
// launch waiting for it.  Every (segment, workgroup) pair has one partial
// row: the workspace holds [2][total workgroups][D] floats.
void build_segment_map(const int64_t *off, const int32_t *mod, int64_t nseg,
                       int64_t G, SegMap *map) {
  const int64_t T = nseg > 0 ? off[nseg] : 0;
  int64_t longest = 0;
  for (int64_t s = 0; s < nseg; ++s)
    longest = std::max(longest, off[s + 1] - off[s]);
  auto workgroups = [&](int64_t R) {
    int64_t n = 0;
    for (int64_t s = 0; s < nseg; ++s) n += (off[s + 1] - off[s] + R - 1) / R;
    return n;
  };
  // R = longest gives one workgroup per non-empty segment, at most 128 <= G
  int64_t lo = std::max<int64_t>(1, (T + G - 1) / G), hi = std::max<int64_t>(1, longest);
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (workgroups(mid) <= G)
      hi = mid;
    else
      lo = mid + 1;
  }
  const int64_t R = lo;
  int64_t wg = 0;
  map->nseg = (int32_t)nseg;
  for (int64_t s = 0; s < nseg; ++s) {
    map->wg_start[s] = (int32_t)wg;
    map->row_start[s] = off[s];
    map->mod[s] = mod ? mod[s] : (int32_t)s;
    wg += (off[s + 1] - off[s] + R - 1) / R;
  }
  map->wg_start[nseg] = (int32_t)wg;
  map->row_start[nseg] = T;
}

bool plan_segments(const int64_t *off, const int32_t *mod, int64_t nseg,
                   int64_t nvec, bool bwd, SegMap *map, StreamPlan *plan) {
  StreamPlan sp;
  if (!choose_stream_plan(1, 1, nvec, bwd, &sp)) return false;
  // (the forward uses only the table's row and vector columns: its grid
  // covers the rows)
  build_segment_map(off, mod, nseg, (int64_t)kCUs * (bwd ? stream_occ(sp) : 1),
                    map);
  *plan = sp;
  return true;
}

}  // namespace adaln

using namespace adaln;

// --------------------------------------------------------------------- ABI

ADALN_API int64_t adaln_max_d(int dtype) {
  if (dtype != ADALN_F32 && dtype != ADALN_BF16) return 0;
  return max_row_vectors() * elems_per_vec(dtype);
}

ADALN_API const char *adaln_strerror(int code) {
  switch (code) {
    case ADALN_OK: return "success";
    case ADALN_ERR_INVALID: return "invalid argument";
    case ADALN_ERR_DTYPE: return "unknown dtype";
    case ADALN_ERR_ALIGN: return "misaligned pointer or D not a multiple of the vector width";
    case ADALN_ERR_WORKSPACE: return "workspace missing or too small";
    case ADALN_ERR_HIP: return "HIP runtime error";
    case ADALN_ERR_UNSUPPORTED: return "D larger than the kernels support";
    default: return "unknown error code";
  }
}

ADALN_API const char *adaln_last_error(void) { return g_msg; }

ADALN_API int64_t adaln_bshape(int64_t S, int64_t m_mem, int64_t m_comp,
                               int32_t p) {
  if (S <= 0 || m_mem < 0 || m_comp < 0 || p < 0)
    return fail(ADALN_ERR_INVALID, "bshape needs S > 0 and non-negative bounds");
  // compute bound floor(m_comp / S^p); S^p beyond int64 makes it 0
  int64_t power = 1;
  bool huge = false;
  for (int32_t i = 0; i < p && !huge; ++i) {
    if (power > INT64_MAX / S)
      huge = true;
    else
      power *= S;
  }
  const int64_t by_compute = huge ? 0 : m_comp / power;
  const int64_t by_memory = m_mem / S;
  const int64_t b = by_memory < by_compute ? by_memory : by_compute;
  ok();
  return b < 1 ? 1 : b;
}

ADALN_API size_t adaln_bwd_workspace_bytes(int64_t B, int64_t N, int64_t D,
                                           int dtype) {
  if (check_shape(B, N, D, dtype) != ADALN_OK) return 0;
  ok();
  return workspace_bytes(B, N, D, dtype);
}

ADALN_API int adaln_fwd(const void *x, const void *scale, const void *shift,
                        void *y, float *mean, float *rstd, int64_t B,
                        int64_t N, int64_t D, int dtype, void *stream) {
  ADALN_TRY(check_shape(B, N, D, dtype));
  const bool rows = B * N > 0;
  ADALN_TRY(check_ptr(x, rows, "x"));
  ADALN_TRY(check_ptr(scale, rows, "scale"));
  ADALN_TRY(check_ptr(shift, rows, "shift"));
  ADALN_TRY(check_ptr(y, rows, "y"));
  ADALN_TRY(check_ptr(mean, rows, "mean"));
  ADALN_TRY(check_ptr(rstd, rows, "rstd"));
  if (!rows) return ok();
  const int64_t nvec = D / elems_per_vec(dtype);
  hipError_t e = hipSuccess;
  StreamPlan sp;
  if (choose_stream_plan(B, N, nvec, false, &sp))
    e = sp.W > 1 ? launch_fwd_wide(dtype, sp, x, scale, shift, y, mean, rstd,
                                   (int32_t)B, (int32_t)N, (int32_t)D,
                                   (hipStream_t)stream)
                 : launch_fwd_rows(dtype, sp.V, x, scale, shift, y, mean,
                                   rstd, (int32_t)B, (int32_t)N, (int32_t)D,
                                   (hipStream_t)stream);
  else
    return fail(ADALN_ERR_UNSUPPORTED, "no forward plan for D=%lld",
                (long long)D);
  if (e != hipSuccess) return hip_fail(e, "adaln_fwd launch");
  return ok();
}

ADALN_API int adaln_bwd_dx(const void *dy, const void *x, const void *scale,
                           const float *mean, const float *rstd, void *dx,
                           int64_t B, int64_t N, int64_t D, int dtype,
                           void *stream) {
  ADALN_TRY(check_shape(B, N, D, dtype));
  const bool rows = B * N > 0;
  ADALN_TRY(check_ptr(dy, rows, "dy"));
  ADALN_TRY(check_ptr(x, rows, "x"));
  ADALN_TRY(check_ptr(scale, rows, "scale"));
  ADALN_TRY(check_ptr(mean, rows, "mean"));
  ADALN_TRY(check_ptr(rstd, rows, "rstd"));
  ADALN_TRY(check_ptr(dx, rows, "dx"));
  if (!rows) return ok();
  RowPlan plan;
  if (!choose_row_plan(D / elems_per_vec(dtype), &plan))
    return fail(ADALN_ERR_UNSUPPORTED, "no row plan for D=%lld", (long long)D);
  const hipError_t e =
      launch_bwd_dx(dtype, plan, dy, x, scale, mean, rstd, dx, B * N,
                    (int32_t)N, (int32_t)D, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "adaln_bwd_dx launch");
  return ok();
}

ADALN_API int adaln_bwd_dmod(const void *dy, const void *x, const float *mean,
                             const float *rstd, float *dscale, float *dshift,
                             void *workspace, size_t workspace_bytes_given,
                             int64_t B, int64_t N, int64_t D, int dtype,
                             void *stream) {
  ADALN_TRY(check_shape(B, N, D, dtype));
  const bool rows = B * N > 0;
  const bool cols = B > 0;
  ADALN_TRY(check_ptr(dy, rows, "dy"));
  ADALN_TRY(check_ptr(x, rows, "x"));
  ADALN_TRY(check_ptr(mean, rows, "mean"));
  ADALN_TRY(check_ptr(rstd, rows, "rstd"));
  ADALN_TRY(check_ptr(dscale, cols, "dscale"));
  ADALN_TRY(check_ptr(dshift, cols, "dshift"));
  if (!cols) return ok();
  const DmodPlan plan = choose_dmod_plan(B, N, D / elems_per_vec(dtype));
  const size_t need = workspace_bytes(B, N, D, dtype);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes_given < need)
      return fail(ADALN_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu%s",
                  need, workspace_bytes_given,
                  workspace == nullptr ? " (NULL)" : "");
    ADALN_TRY(check_ptr(workspace, true, "workspace"));
  }
  float *part_scale = static_cast<float *>(workspace);
  float *part_shift =
      plan.n_tiles > 0 ? part_scale + (size_t)B * plan.n_tiles * D : nullptr;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (plan.n_tiles > 0)
    e = launch_dmod_partial(dtype, plan, dy, x, mean, rstd, part_scale,
                            part_shift, (int32_t)B, (int32_t)N, (int32_t)D, s);
  if (e == hipSuccess)
    e = launch_dmod_finish(part_scale, part_shift, dscale, dshift, (int32_t)B,
                           (int32_t)D, (int32_t)plan.n_tiles, s);
  if (e != hipSuccess) return hip_fail(e, "adaln_bwd_dmod launch");
  return ok();
}

namespace {

// Workspace check shared by the backward entry points.
int check_workspace(const void *workspace, size_t given, size_t need) {
  if (need > 0 && (workspace == nullptr || given < need))
    return fail(ADALN_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu%s",
                need, given, workspace == nullptr ? " (NULL)" : "");
  return check_ptr(workspace, need > 0, "workspace");
}

}  // namespace

ADALN_API int adaln_bwd_fused(const void *dy, const void *x, const void *scale,
                              const float *mean, const float *rstd, void *dx,
                              void *workspace, size_t workspace_bytes_given,
                              int64_t B, int64_t N, int64_t D, int dtype,
                              void *stream) {
  ADALN_TRY(check_shape(B, N, D, dtype));
  const bool rows = B * N > 0;
  ADALN_TRY(check_ptr(dy, rows, "dy"));
  ADALN_TRY(check_ptr(x, rows, "x"));
  ADALN_TRY(check_ptr(scale, rows, "scale"));
  ADALN_TRY(check_ptr(mean, rows, "mean"));
  ADALN_TRY(check_ptr(rstd, rows, "rstd"));
  ADALN_TRY(check_ptr(dx, rows, "dx"));
  StreamPlan plan;
  if (!choose_stream_plan(B, N, D / elems_per_vec(dtype), true, &plan))
    return fail(ADALN_ERR_UNSUPPORTED,
                "D=%lld is too wide for the fused backward", (long long)D);
  ADALN_TRY(check_workspace(workspace, workspace_bytes_given,
                            workspace_bytes(B, N, D, dtype)));
  if (!rows) return ok();
  float *part_scale = static_cast<float *>(workspace);
  float *part_shift = part_scale + (size_t)B * plan.bps * D;
  const hipError_t e =
      plan.W > 1
          ? launch_bwd_wide(dtype, plan, dy, x, scale, mean, rstd, dx,
                            part_scale, part_shift, (int32_t)B, (int32_t)N,
                            (int32_t)D, (hipStream_t)stream)
          : launch_bwd_fused(dtype, plan, dy, x, scale, mean, rstd, dx,
                             part_scale, part_shift, (int32_t)B, (int32_t)N,
                             (int32_t)D, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "adaln_bwd_fused launch");
  return ok();
}

ADALN_API int adaln_bwd_fused_plan(int64_t B, int64_t N, int64_t D,
                                   int dtype, int64_t *out) {
  ADALN_TRY(check_shape(B, N, D, dtype));
  if (out == nullptr) return fail(ADALN_ERR_INVALID, "out is NULL");
  StreamPlan plan;
  if (!choose_stream_plan(B, N, D / elems_per_vec(dtype), true, &plan))
    return fail(ADALN_ERR_UNSUPPORTED,
                "D=%lld is too wide for the fused backward", (long long)D);
  out[0] = plan.V;
  out[1] = plan.W;
  out[2] = plan.grid;
  out[3] = plan.bps;
  return ok();
}

ADALN_API int adaln_plan(int which, int64_t B, int64_t N, int64_t D,
                         int dtype, int64_t *out) {
  ADALN_TRY(check_shape(B, N, D, dtype));
  if (out == nullptr) return fail(ADALN_ERR_INVALID, "out is NULL");
  if (which < 0 || which > 3)
    return fail(ADALN_ERR_INVALID,
                "which must be 0 (forward), 1 (fused backward), 2 (finish) "
                "or 3 (D-tile grid), got %d",
                which);
  const int64_t nvec = D / elems_per_vec(dtype);
  StreamPlan sp;
  if (which == 3) {
    const DmodPlan dp = choose_dmod_plan(B, N, nvec);
    const int64_t v[7] = {dp.d_tiles, dp.n_tile, dp.n_tiles,
                          (int64_t)dp.d_tiles * dp.n_tiles * B, 256, 0, 0};
    std::copy(v, v + 7, out);
    return ok();
  }
  if (which == 2) {
    // the partial rows each output sums: the fused plan's workgroups per
    // sample, or the D-tile plan's tiles for rows too wide for it
    const int64_t rows = choose_stream_plan(B, N, nvec, true, &sp)
                             ? (B > 0 && N > 0 ? sp.bps : 0)
                             : choose_dmod_plan(B, N, nvec).n_tiles;
    const FinishPlan fp = finish_plan(B, (int32_t)D, rows);
    const int64_t launched = fp.blocks < kMaxGrid ? fp.blocks : kMaxGrid;
    const int64_t v[7] = {fp.F, fp.wpc, fp.cpb, B > 0 ? launched : 0,
                          fp.threads, rows, 0};
    std::copy(v, v + 7, out);
    return ok();
  }
  if (choose_stream_plan(B, N, nvec, which == 1, &sp)) {
    const int64_t walkers = rows_per_workgroup(sp.W);
    const int64_t v[7] = {sp.V,      sp.W,    sp.grid, sp.bps,
                          sp.groups, walkers, sp.skew};
    std::copy(v, v + 7, out);
  } else {
    return fail(ADALN_ERR_UNSUPPORTED, "no %s plan for D=%lld",
                which ? "fused backward" : "forward", (long long)D);
  }
  return ok();
}

ADALN_API int adaln_bwd_finish(const void *workspace,
                               size_t workspace_bytes_given, float *dscale,
                               float *dshift, int64_t B, int64_t N, int64_t D,
                               int dtype, void *stream) {
  ADALN_TRY(check_shape(B, N, D, dtype));
  ADALN_TRY(check_ptr(dscale, B > 0, "dscale"));
  ADALN_TRY(check_ptr(dshift, B > 0, "dshift"));
  StreamPlan plan;
  if (!choose_stream_plan(B, N, D / elems_per_vec(dtype), true, &plan))
    return fail(ADALN_ERR_UNSUPPORTED,
                "D=%lld is too wide for the fused backward", (long long)D);
  ADALN_TRY(check_workspace(workspace, workspace_bytes_given,
                            workspace_bytes(B, N, D, dtype)));
  if (B == 0) return ok();
  const float *part_scale = static_cast<const float *>(workspace);
  const float *part_shift =
      plan.bps > 0 ? part_scale + (size_t)B * plan.bps * D : nullptr;
  const hipError_t e =
      launch_dmod_finish(part_scale, part_shift, dscale, dshift, (int32_t)B,
                         (int32_t)D, (int32_t)plan.bps, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "adaln_bwd_finish launch");
  return ok();
}

ADALN_API int adaln_bwd(const void *dy, const void *x, const void *scale,
                        const float *mean, const float *rstd, void *dx,
                        float *dscale, float *dshift, void *workspace,
                        size_t workspace_bytes_given, int64_t B, int64_t N,
                        int64_t D, int dtype, void *stream) {
  // every check of both launches runs before either is enqueued
  ADALN_TRY(check_shape(B, N, D, dtype));
  const bool rows = B * N > 0;
  ADALN_TRY(check_ptr(dy, rows, "dy"));
  ADALN_TRY(check_ptr(x, rows, "x"));
  ADALN_TRY(check_ptr(scale, rows, "scale"));
  ADALN_TRY(check_ptr(mean, rows, "mean"));
  ADALN_TRY(check_ptr(rstd, rows, "rstd"));
  ADALN_TRY(check_ptr(dx, rows, "dx"));
  ADALN_TRY(check_ptr(dscale, B > 0, "dscale"));
  ADALN_TRY(check_ptr(dshift, B > 0, "dshift"));
  ADALN_TRY(check_workspace(workspace, workspace_bytes_given,
                            workspace_bytes(B, N, D, dtype)));
  // every row width that check_shape admits has a fused plan
  ADALN_TRY(adaln_bwd_fused(dy, x, scale, mean, rstd, dx, workspace,
                            workspace_bytes_given, B, N, D, dtype, stream));
  return adaln_bwd_finish(workspace, workspace_bytes_given, dscale, dshift, B,
                          N, D, dtype, stream);
}

// ------------------------------------------------------ packed segments

namespace {

// Validates the segment table (host arrays) and the shape.
int check_segments(const int64_t *off, const int32_t *mod, int64_t nseg,
                   int64_t nmod, int64_t D, int dtype) {
  ADALN_TRY(check_shape(1, 0, D, dtype));
  if (nseg < 0 || nseg > kMaxSegments)
    return fail(ADALN_ERR_INVALID, "nseg=%lld outside [0, %d]",
                (long long)nseg, kMaxSegments);
  if (nmod < 0 || nmod > kMaxB)
    return fail(ADALN_ERR_INVALID, "nmod=%lld is invalid", (long long)nmod);
  if (nseg == 0) return ADALN_OK;
  if (off == nullptr) return fail(ADALN_ERR_INVALID, "seg_offsets is NULL");
  if (off[0] != 0) return fail(ADALN_ERR_INVALID, "seg_offsets[0] must be 0");
  for (int64_t s = 0; s < nseg; ++s) {
    if (off[s + 1] < off[s])
      return fail(ADALN_ERR_INVALID, "seg_offsets decrease at %lld",
                  (long long)s);
    const int64_t m = mod ? mod[s] : s;
    if (m < 0 || m >= nmod)
      return fail(ADALN_ERR_INVALID,
                  "segment %lld uses modulation vector %lld of %lld",
                  (long long)s, (long long)m, (long long)nmod);
  }
  if (off[nseg] > kMaxRows)
    return fail(ADALN_ERR_INVALID, "more than 2^31-1 rows");
  if (nmod > kMaxRows / D) return fail(ADALN_ERR_INVALID, "nmod*D too large");
  return ADALN_OK;
}

}  // namespace

ADALN_API size_t adaln_bwd_segments_workspace_bytes(const int64_t *seg_offsets,
                                                    int64_t nseg, int64_t D,
                                                    int dtype) {
  if (check_segments(seg_offsets, nullptr, nseg, nseg > 0 ? nseg : 1, D,
                     dtype) != ADALN_OK)
    return 0;
  SegMap map;
  StreamPlan sp;
  if (!plan_segments(seg_offsets, nullptr, nseg, D / elems_per_vec(dtype),
                     true, &map, &sp))
    return 0;
  ok();
  return partial_bytes(map.wg_start[nseg], 1, D);
}

ADALN_API int adaln_fwd_segments(const void *x, const void *scale,
                                 const void *shift, void *y, float *mean,
                                 float *rstd, const int64_t *seg_offsets,
                                 const int32_t *seg_mod, int64_t nseg,
                                 int64_t nmod, int64_t D, int dtype,
                                 void *stream) {
  ADALN_TRY(check_segments(seg_offsets, seg_mod, nseg, nmod, D, dtype));
  const int64_t T = nseg > 0 ? seg_offsets[nseg] : 0;
  const bool rows = T > 0;
  ADALN_TRY(check_ptr(x, rows, "x"));
  ADALN_TRY(check_ptr(scale, rows, "scale"));
  ADALN_TRY(check_ptr(shift, rows, "shift"));
  ADALN_TRY(check_ptr(y, rows, "y"));
  ADALN_TRY(check_ptr(mean, rows, "mean"));
  ADALN_TRY(check_ptr(rstd, rows, "rstd"));
  const int64_t nvec = D / elems_per_vec(dtype);
  SegMap map;
  StreamPlan sp;
  hipError_t e = hipSuccess;
  if (plan_segments(seg_offsets, seg_mod, nseg, nvec, false, &map, &sp)) {
    if (!rows) return ok();
    e = sp.W > 1 ? launch_fwd_wide_segments(dtype, sp, map, x, scale, shift,
                                            y, mean, rstd, (int32_t)D,
                                            (hipStream_t)stream)
                 : launch_fwd_segments(dtype, sp.V, map, x, scale, shift, y,
                                       mean, rstd, (int32_t)D,
                                       (hipStream_t)stream);
  } else {
    return fail(ADALN_ERR_UNSUPPORTED,
                "D=%lld is too wide for the segment kernels", (long long)D);
  }
  if (e != hipSuccess) return hip_fail(e, "adaln_fwd_segments launch");
  return ok();
}

ADALN_API int adaln_bwd_segments(const void *dy, const void *x,
                                 const void *scale, const float *mean,
                                 const float *rstd, void *dx, float *dscale,
                                 float *dshift, void *workspace,
                                 size_t workspace_bytes_given,
                                 const int64_t *seg_offsets,
                                 const int32_t *seg_mod, int64_t nseg,
                                 int64_t nmod, int64_t D, int dtype,
                                 void *stream) {
  ADALN_TRY(check_segments(seg_offsets, seg_mod, nseg, nmod, D, dtype));
  const int64_t T = nseg > 0 ? seg_offsets[nseg] : 0;
  const bool rows = T > 0;
  ADALN_TRY(check_ptr(dy, rows, "dy"));
  ADALN_TRY(check_ptr(x, rows, "x"));
  ADALN_TRY(check_ptr(scale, rows, "scale"));
  ADALN_TRY(check_ptr(mean, rows, "mean"));
  ADALN_TRY(check_ptr(rstd, rows, "rstd"));
  ADALN_TRY(check_ptr(dx, rows, "dx"));
  ADALN_TRY(check_ptr(dscale, nmod > 0, "dscale"));
  ADALN_TRY(check_ptr(dshift, nmod > 0, "dshift"));
  SegMap map;
  StreamPlan sp;
  if (!plan_segments(seg_offsets, seg_mod, nseg, D / elems_per_vec(dtype),
                     true, &map, &sp))
    return fail(ADALN_ERR_UNSUPPORTED,
                "D=%lld is too wide for the segment kernels", (long long)D);
  const size_t need = partial_bytes(map.wg_start[nseg], 1, D);
  ADALN_TRY(check_workspace(workspace, workspace_bytes_given, need));
  if (nmod == 0) return ok();
  float *part_scale = static_cast<float *>(workspace);
  float *part_shift = part_scale + (size_t)map.wg_start[nseg] * D;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (rows)
    e = sp.W > 1 ? launch_bwd_wide_segments(dtype, sp, map, dy, x, scale,
                                            mean, rstd, dx, part_scale,
                                            part_shift, (int32_t)D, s)
                 : launch_bwd_segments(dtype, sp.V, map, dy, x, scale, mean,
                                       rstd, dx, part_scale, part_shift,
                                       (int32_t)D, s);
  if (e == hipSuccess)
    e = launch_finish_segments(part_scale, part_shift, dscale, dshift, map,
                               (int32_t)nmod, (int32_t)D, s);
  if (e != hipSuccess) return hip_fail(e, "adaln_bwd_segments launch");
  return ok();
}

// ------------------------------------------------- backward without a buffer

namespace {

// Scratch of adaln_bwd_noalloc: the backward's partial rows, in a device
// array of the library's own.  Each GPU the library runs on holds its own
// copy until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device memory: the device address is looked up once
// per device with hipGetSymbolAddress and only that address is passed on.
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices] = {};

// Device address of the calling thread's current device's scratch.
int scratch_address(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "adaln_bwd_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ADALN_ERR_HIP, "adaln_bwd_noalloc: device %d out of range",
                dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess)
      return hip_fail(e, "adaln_bwd_noalloc: hipGetSymbolAddress");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return ADALN_OK;
}

}  // namespace

ADALN_API int adaln_bwd_noalloc(const void *dy, const void *x,
                                const void *scale, const float *mean,
                                const float *rstd, void *dx, float *dscale,
                                float *dshift, int64_t B, int64_t N,
                                int64_t D, int dtype, void *stream) {
  // the checks of adaln_bwd, then the size check, before any HIP call
  ADALN_TRY(check_shape(B, N, D, dtype));
  const bool rows = B * N > 0;
  ADALN_TRY(check_ptr(dy, rows, "dy"));
  ADALN_TRY(check_ptr(x, rows, "x"));
  ADALN_TRY(check_ptr(scale, rows, "scale"));
  ADALN_TRY(check_ptr(mean, rows, "mean"));
  ADALN_TRY(check_ptr(rstd, rows, "rstd"));
  ADALN_TRY(check_ptr(dx, rows, "dx"));
  ADALN_TRY(check_ptr(dscale, B > 0, "dscale"));
  ADALN_TRY(check_ptr(dshift, B > 0, "dshift"));
  const size_t need = workspace_bytes(B, N, D, dtype);
  if (need > kScratchBytes)
    return fail(ADALN_ERR_WORKSPACE,
                "adaln_bwd_noalloc: this shape needs %zu bytes of scratch, "
                "the library's static scratch holds %zu (use adaln_bwd with "
                "a workspace)",
                need, kScratchBytes);
  if (B == 0) return ok();
  void *ws = nullptr;
  ADALN_TRY(scratch_address(&ws));
  return adaln_bwd(dy, x, scale, mean, rstd, dx, dscale, dshift, ws,
                   kScratchBytes, B, N, D, dtype, stream);
}
