// Forward kernels of the fused AdaLN operator (AdaptiveLoad technical
// summary, section 2.B, forward pass): per token row, mean and variance over
// D, then y = xhat * (1 + scale[b]) + shift[b], with x read from HBM once and
// y written once, in a single launch.
//
// fwd_rows_kernel (rows of up to 1024 16-byte vectors): one wavefront per
// row, lane l holding vectors k*64 + l, k < V, in registers; no barrier and
// no loop.  The grid covers the rows of the call: wavefront w of workgroup g
// takes row first + 4g + w (one launch per 2^22 rows).  A wavefront issues
// the loads of its row first, then finds its row's modulation vector (the
// sample r / N, or the packed segment holding r) and loads its scale and
// shift (L2 hits after the first rows of a sample).  Mean and variance are
// two-pass over the register-resident row (DPP reductions).
//
// No occupancy is imposed: with short-lived wavefronts the hardware keeps as
// many rows in flight as the registers allow, and the rows in flight at any
// time are the consecutive rows the dispatcher has reached, one window over
// memory for any number of samples.  Measured on MI355X against a persistent
// grid (a fixed number of workgroups per CU walking each sample's rows with
// scale and shift kept in registers), in one process on the same buffers,
// bf16: 16 x 1560 x 1536 30.5 -> 27.2 us, 84 x 1560 x 3072 307 -> 267 us,
// 256 x 256 x 1152 61.6 -> 53.0 us, 1 x 75600 x 5120 264 -> 256 us.  The same
// kernel walking rows inside the work map's loops kept more registers alive
// (one wavefront per SIMD at 640 vectors instead of two) and lost most of it.
//
// Wider rows: fwd_wide_kernel (fwd_wide.hip).
//
// All sums run in a fixed order, so results are reproducible bit for bit.
#include "common.hpp"
#include "launch.hpp"

namespace adaln {

template <typename T, int V, bool FULL, class Map>
__global__ __launch_bounds__(kBlock) void fwd_rows_kernel(
    const T *__restrict__ x, const T *__restrict__ scale,
    const T *__restrict__ shift, T *__restrict__ y, float *__restrict__ mean,
    float *__restrict__ rstd, int32_t D, int64_t first, int64_t end,
    Map map) {
  constexpr int E = Elems<T>::value;
  const int lane = lane_id();
  const int64_t r = first + (int64_t)blockIdx.x * (kBlock / kWave) + wave_id();
  if (r >= end) return;
  const int nvec = D / E;
  const float inv_d = 1.0f / (float)D;

  int jv[V], jl[V];  // vector of lane l, and the vector its load reads
  bool ok[V];
#pragma unroll
  for (int k = 0; k < V; ++k) {
    jv[k] = k * kWave + lane;
    ok[k] = FULL || jv[k] < nvec;
    jl[k] = FULL ? jv[k] : clamp_vec(jv[k], nvec);
  }
  const int64_t off = r * D;
  Vec xv[V], sv[V], hv[V];
#pragma unroll
  for (int k = 0; k < V; ++k)
    xv[k] = load_stream(x + off + (int64_t)jl[k] * E);
  const int64_t mod = row_mod(map, r);
#pragma unroll
  for (int k = 0; k < V; ++k) {
    const int64_t c = mod * D + (int64_t)jl[k] * E;
    sv[k] = load_vec(scale + c);
    hv[k] = load_vec(shift + c);
  }
  if constexpr (!FULL) mask_tail(xv, ok);
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < V; ++k)
#pragma unroll
    for (int e = 0; e < E; ++e) s += elem<T>(xv[k], e);
  const float mu = wave_sum(s) * inv_d;
  if constexpr (fwd_rows_rewiden(V, E)) {
#pragma unroll
    for (int k = 0; k < V; ++k) opaque(xv[k]);
  }
  float q = 0.f;
#pragma unroll
  for (int k = 0; k < V; ++k) {
    if (ok[k]) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float c = elem<T>(xv[k], e) - mu;
        q = fmaf(c, c, q);
      }
    }
  }
  const float rs = 1.0f / sqrtf(wave_sum(q) * inv_d + kEps);
  if (lane == 0) {
    mean[r] = mu;
    rstd[r] = rs;
  }
  if constexpr (fwd_rows_rewiden(V, E)) {
#pragma unroll
    for (int k = 0; k < V; ++k) opaque(xv[k]), opaque(sv[k]), opaque(hv[k]);
  }
#pragma unroll
  for (int k = 0; k < V; ++k) {
    if (ok[k]) {
      float o[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float xh = (elem<T>(xv[k], e) - mu) * rs;
        o[e] = fmaf(xh, 1.0f + elem<T>(sv[k], e), elem<T>(hv[k], e));
      }
      store_stream(y + off + (int64_t)jv[k] * E, pack<T>(o));
    }
  }
}

namespace {

// Rows per launch: kMaxGrid four-wavefront workgroups, one row each.
constexpr int64_t kRowsPerLaunch = kMaxGrid * (kBlock / kWave);

template <typename T, int V, bool FULL, class Map>
hipError_t fwd_rows_v(int64_t rows, const Map &map, const void *x,
                      const void *scale, const void *shift, void *y,
                      float *mean, float *rstd, int32_t D, hipStream_t s) {
  for (int64_t first = 0; first < rows; first += kRowsPerLaunch) {
    const int64_t end =
        rows - first < kRowsPerLaunch ? rows : first + kRowsPerLaunch;
    const hipError_t e = launch_kernel(
        fwd_rows_kernel<T, V, FULL, Map>, (end - first + 3) / 4, s,
        (const T *)x, (const T *)scale, (const T *)shift, (T *)y, mean, rstd,
        D, first, end, map);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

#define ADALN_FWD_ROWS_CASE(V_)                                              \
  if (V == V_) {                                                             \
    if (full)                                                                \
      return dtype == 1 ? fwd_rows_v<bf16, V_, true>(rows, map, x, scale,    \
                                                     shift, y, mean, rstd,   \
                                                     D, stream)              \
                        : fwd_rows_v<float, V_, true>(rows, map, x, scale,   \
                                                      shift, y, mean, rstd,  \
                                                      D, stream);            \
    return dtype == 1 ? fwd_rows_v<bf16, V_, false>(rows, map, x, scale,     \
                                                    shift, y, mean, rstd, D, \
                                                    stream)                  \
                      : fwd_rows_v<float, V_, false>(rows, map, x, scale,    \
                                                     shift, y, mean, rstd,   \
                                                     D, stream);             \
  }

namespace {

template <class Map>
hipError_t fwd_rows_dispatch(int dtype, int V, int64_t rows, const Map &map,
                             const void *x, const void *scale,
                             const void *shift, void *y, float *mean,
                             float *rstd, int32_t D, hipStream_t stream) {
  const int E = dtype == 1 ? 8 : 4;
  const bool full = (int64_t)V * kWave * E == D;
  ADALN_STREAM_V(ADALN_FWD_ROWS_CASE)
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fwd_rows(int dtype, int V, const void *x, const void *scale,
                           const void *shift, void *y, float *mean,
                           float *rstd, int32_t B, int32_t N, int32_t D,
                           hipStream_t stream) {
  return fwd_rows_dispatch(dtype, V, (int64_t)B * N, BatchRows{N}, x, scale,
                           shift, y, mean, rstd, D, stream);
}

hipError_t launch_fwd_segments(int dtype, int V, const SegMap &map,
                               const void *x, const void *scale,
                               const void *shift, void *y, float *mean,
                               float *rstd, int32_t D, hipStream_t stream) {
  return fwd_rows_dispatch(dtype, V, map.row_start[map.nseg], map, x, scale,
                           shift, y, mean, rstd, D, stream);
}

}  // namespace adaln
