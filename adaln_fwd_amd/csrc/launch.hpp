// Internal launch interface between the C ABI (abi.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <type_traits>

namespace adaln {

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

// The fused backward: a workgroup of W wavefronts owns n_tile token rows of
// one sample; each lane holds V vectors of a row.  ADALN_FUSED_V lists the
// instantiated V.
#define ADALN_FUSED_V(X) X(1) X(2) X(3) X(4)

struct FusedPlan {
  int V = 0;
  int W = 0;
  int n_tile = 0;
  int n_tiles = 0;
};

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
bool choose_fused_plan(int64_t B, int64_t N, int64_t nvec, FusedPlan *plan);

// Launchers: enqueue on `stream`, return hipGetLastError() of the launch.
hipError_t launch_fwd(int dtype, const RowPlan &plan, const void *x,
                      const void *scale, const void *shift, void *y,
                      float *mean, float *rstd, int64_t rows, int32_t N,
                      int32_t D, hipStream_t stream);

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

// dscale/dshift = sums over n_tiles of [B, n_tiles, D] partials, in index
// order (zero when n_tiles == 0).
hipError_t launch_dmod_finish(const float *part_scale,
                              const float *part_shift, float *dscale,
                              float *dshift, int32_t B, int32_t D,
                              int32_t n_tiles, hipStream_t stream);

hipError_t launch_bwd_fused(int dtype, const FusedPlan &plan, const void *dy,
                            const void *x, const void *scale,
                            const float *mean, const float *rstd, void *dx,
                            float *part_scale, float *part_shift, int32_t B,
                            int32_t N, int32_t D, hipStream_t stream);

}  // namespace adaln
