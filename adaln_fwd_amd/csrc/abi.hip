// C ABI of the fused AdaLN library: argument validation, launch planning and
// dispatch.  Declarations, layouts and error behaviour are documented in
// include/adaln.h.  Every check runs on the host before any HIP call, so an
// invalid call enqueues nothing.
#include <stdarg.h>
#include <stdio.h>
#include <stdint.h>

#include "../../include/adaln.h"
#include "launch.hpp"

#define ADALN_API extern "C" __attribute__((visibility("default")))

namespace adaln {
namespace {

thread_local char g_msg[256] = "";

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
  FusedPlan fp;
  const size_t a = partial_bytes(dp.n_tiles, B, D);
  const size_t b = choose_fused_plan(B, N, nvec, &fp)
                       ? partial_bytes(fp.n_tiles, B, D)
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

// The fused backward.  V is the smallest number of vectors per lane (at most
// 4) that lets at most 8 wavefronts hold a row: small V keeps the per-lane
// accumulators (2*V*E floats) in registers.  Wider rows (more than 2048
// vectors) have no fused plan and take the dx + D-tile kernels instead.  n_tile
// aims at about ADALN_FUSED_TARGET_WAVES wavefronts over the whole grid and
// is at least 16 rows, since each tile writes 8 bytes of partials per
// feature.
#ifndef ADALN_FUSED_TARGET_WAVES
#define ADALN_FUSED_TARGET_WAVES 2048
#endif

bool choose_fused_plan(int64_t B, int64_t N, int64_t nvec, FusedPlan *plan) {
  FusedPlan p;
  for (int v = 1; v <= 4 && p.V == 0; ++v) {
    const int64_t w = (nvec + 64 * v - 1) / (64 * v);
    if (w <= 8) {
      p.V = v;
      p.W = (int)w;
    }
  }
  if (p.V == 0) return false;
  if (B > 0 && N > 0) {
    int64_t target_blocks = ADALN_FUSED_TARGET_WAVES / p.W;
    if (target_blocks < 1) target_blocks = 1;
    int64_t tiles_per_sample = (target_blocks + B - 1) / B;
    int64_t n_tile = (N + tiles_per_sample - 1) / tiles_per_sample;
    if (n_tile < 16) n_tile = 16;
    p.n_tile = (int)n_tile;
    p.n_tiles = (int)((N + n_tile - 1) / n_tile);
  }
  *plan = p;
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
  RowPlan plan;
  if (!choose_row_plan(D / elems_per_vec(dtype), &plan))
    return fail(ADALN_ERR_UNSUPPORTED, "no row plan for D=%lld", (long long)D);
  const hipError_t e =
      launch_fwd(dtype, plan, x, scale, shift, y, mean, rstd, B * N,
                 (int32_t)N, (int32_t)D, (hipStream_t)stream);
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
  FusedPlan plan;
  if (!choose_fused_plan(B, N, D / elems_per_vec(dtype), &plan))
    return fail(ADALN_ERR_UNSUPPORTED,
                "D=%lld is too wide for the fused backward", (long long)D);
  ADALN_TRY(check_workspace(workspace, workspace_bytes_given,
                            workspace_bytes(B, N, D, dtype)));
  if (!rows) return ok();
  float *part_scale = static_cast<float *>(workspace);
  float *part_shift = part_scale + (size_t)B * plan.n_tiles * D;
  const hipError_t e = launch_bwd_fused(
      dtype, plan, dy, x, scale, mean, rstd, dx, part_scale, part_shift,
      (int32_t)B, (int32_t)N, (int32_t)D, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "adaln_bwd_fused launch");
  return ok();
}

ADALN_API int adaln_bwd_fused_plan(int64_t B, int64_t N, int64_t D,
                                   int dtype, int64_t *out) {
  ADALN_TRY(check_shape(B, N, D, dtype));
  if (out == nullptr) return fail(ADALN_ERR_INVALID, "out is NULL");
  FusedPlan plan;
  if (!choose_fused_plan(B, N, D / elems_per_vec(dtype), &plan))
    return fail(ADALN_ERR_UNSUPPORTED,
                "D=%lld is too wide for the fused backward", (long long)D);
  out[0] = plan.V;
  out[1] = plan.W;
  out[2] = plan.n_tile;
  out[3] = plan.n_tiles;
  return ok();
}

ADALN_API int adaln_bwd_finish(const void *workspace,
                               size_t workspace_bytes_given, float *dscale,
                               float *dshift, int64_t B, int64_t N, int64_t D,
                               int dtype, void *stream) {
  ADALN_TRY(check_shape(B, N, D, dtype));
  ADALN_TRY(check_ptr(dscale, B > 0, "dscale"));
  ADALN_TRY(check_ptr(dshift, B > 0, "dshift"));
  FusedPlan plan;
  if (!choose_fused_plan(B, N, D / elems_per_vec(dtype), &plan))
    return fail(ADALN_ERR_UNSUPPORTED,
                "D=%lld is too wide for the fused backward", (long long)D);
  ADALN_TRY(check_workspace(workspace, workspace_bytes_given,
                            workspace_bytes(B, N, D, dtype)));
  if (B == 0) return ok();
  const float *part_scale = static_cast<const float *>(workspace);
  const float *part_shift =
      plan.n_tiles > 0 ? part_scale + (size_t)B * plan.n_tiles * D : nullptr;
  const hipError_t e =
      launch_dmod_finish(part_scale, part_shift, dscale, dshift, (int32_t)B,
                         (int32_t)D, (int32_t)plan.n_tiles,
                         (hipStream_t)stream);
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
  FusedPlan plan;
  if (choose_fused_plan(B, N, D / elems_per_vec(dtype), &plan)) {
    ADALN_TRY(adaln_bwd_fused(dy, x, scale, mean, rstd, dx, workspace,
                              workspace_bytes_given, B, N, D, dtype, stream));
    return adaln_bwd_finish(workspace, workspace_bytes_given, dscale, dshift,
                            B, N, D, dtype, stream);
  }
  // rows too wide for the fused kernel: dx, then the D-tile reduction
  ADALN_TRY(adaln_bwd_dx(dy, x, scale, mean, rstd, dx, B, N, D, dtype, stream));
  return adaln_bwd_dmod(dy, x, mean, rstd, dscale, dshift, workspace,
                        workspace_bytes_given, B, N, D, dtype, stream);
}
