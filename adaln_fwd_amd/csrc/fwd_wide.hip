// Forward of the fused AdaLN operator for rows of 1025 to 4096 16-byte
// vectors (bf16 D of 8200 to 32768, f32 D of 4100 to 16384): per row, mean
// and variance over D, then y = xhat * (1 + scale[b]) + shift[b], as in
// fwd_rows_kernel (AdaptiveLoad technical summary, section 2.B, forward
// pass), with each row split between W = 2 or 4 wavefronts.
//
// A row of more than 1024 vectors does not fit one wavefront's registers
// next to the modulation vectors.  As in the wide backward, the four
// wavefronts of a workgroup form 4 / W row groups (two pairs, or one quad);
// wavefront h of a group owns the contiguous vectors [h*V*64, (h+1)*V*64) of
// the group's row (lane l: vector (h*V + k)*64 + l).  Like fwd_rows_kernel,
// the grid covers the rows of the call with no loop and no imposed
// occupancy: row group j of workgroup g takes row first + (4/W)*g + j (one
// launch per 2^20 workgroups), loads its part of the row, then finds the
// row's modulation vector and loads its part of scale and shift.  Each
// wavefront reduces its part with DPP to a sum and a centred sum of squares
// around the part's own mean; lane 0 stores the two values, one barrier,
// and every wavefront of the group combines the W parts in part order with
// the pairwise update of Chan, Golub and LeVeque (1979),
//     mean = sum_h S_h / D,  M2 = sum_h (M2_h + n_h * (S_h / n_h - mean)^2),
// which keeps the accuracy of a two-pass variance.  All sums run in a fixed
// order: results are reproducible bit for bit.
//
// Measured on MI355X against a persistent grid at one wavefront per SIMD
// with the next row in flight (scale and shift kept in registers), in one
// process on the same buffers: bf16 1 x 8192 x 32768 226.9 -> 183.4 us,
// 1 x 16384 x 12288 150.1 -> 132.6 us, 16 x 1560 x 12288 241.5 -> 203.5 us,
// 2 x 8000 x 12296 223.7 -> 161.9 us, 84 x 300 x 16384 331.6 -> 281.1 us;
// f32 1 x 30000 x 6148 321.3 -> 295.2 us, 1 x 16384 x 12288 283.6 -> 268.1
// us, and 0.5-4.9% slower only for f32 rows of 16 vectors per lane (D =
// 16384).  The same grid written inside the work map's walk loops kept more
// registers alive and was 3-12% slower than the persistent kernel.  Ragged
// f32 rows of 16 vectors per lane load scale and shift late
// (fwd_wide_late_mod in launch.hpp).
#include "common.hpp"
#include "launch.hpp"

namespace adaln {

template <typename T, int V, int W, bool FULL, class Map>
__global__ __launch_bounds__(kBlock) void fwd_wide_kernel(
    const T *__restrict__ x, const T *__restrict__ scale,
    const T *__restrict__ shift, T *__restrict__ y, float *__restrict__ mean,
    float *__restrict__ rstd, int32_t D, int64_t first, int64_t end,
    Map map) {
  static_assert(W == 2 || W == 4, "a row takes two or four wavefronts");
  constexpr int E = Elems<T>::value;
  constexpr int kRows = kBlock / kWave / W;  // rows a workgroup works on
  __shared__ float red[kRows][W][2];          // [group][part][sum, m2]
  const int lane = lane_id();
  const int wave = wave_id();
  const int group = wave / W;  // row group (pair or quad) of this wavefront
  const int part = wave % W;   // its part of the group's row
  const int nvec = D / E;
  const float inv_d = 1.0f / (float)D;
  const int64_t r = first + (int64_t)blockIdx.x * kRows + group;
  // a group past the last row still takes part in the barrier; it reads
  // the last row (in bounds) and writes nothing
  const bool live = r < end;  // uniform across the wavefront
  const int64_t rr = live ? r : end - 1;

  int jv[V], jl[V];  // vector of lane l, and the vector its load reads
  bool ok[V];
#pragma unroll
  for (int k = 0; k < V; ++k) {
    jv[k] = (part * V + k) * kWave + lane;
    ok[k] = FULL || jv[k] < nvec;
    jl[k] = FULL ? jv[k] : clamp_vec(jv[k], nvec);
  }
  // elements of the row that part h holds (the same in every wavefront)
  auto count = [&](int h) -> float {
    const int held =
        FULL ? V * kWave : max(0, min(V * kWave, nvec - h * V * kWave));
    return (float)(held * E);
  };

  const int64_t off = rr * D;
  Vec xv[V], sv[V], hv[V];
#pragma unroll
  for (int k = 0; k < V; ++k)
    xv[k] = load_stream(x + off + (int64_t)jl[k] * E);
  const int64_t mod = row_mod(map, rr);
  constexpr bool kLate = fwd_wide_late_mod(V, E, FULL);
  if constexpr (!kLate) {
#pragma unroll
    for (int k = 0; k < V; ++k) {
      const int64_t c = mod * D + (int64_t)jl[k] * E;
      sv[k] = load_vec(scale + c);
      hv[k] = load_vec(shift + c);
    }
  }
  if constexpr (!FULL) mask_tail(xv, ok);

  // this part's sum, and its centred sum of squares around its mean
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < V; ++k)
#pragma unroll
    for (int e = 0; e < E; ++e) s += elem<T>(xv[k], e);
  const float cnt_w = count(part);
  const float sum_w = wave_sum(s);
  const float mean_w = cnt_w > 0.f ? sum_w / cnt_w : 0.f;
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
        const float c = elem<T>(xv[k], e) - mean_w;
        q = fmaf(c, c, q);
      }
    }
  }
  const float m2_w = wave_sum(q);
  if (lane == 0) {
    red[group][part][0] = sum_w;
    red[group][part][1] = m2_w;
  }
  __syncthreads();
  if (!live) return;
  float tot = red[group][0][0];
#pragma unroll
  for (int h = 1; h < W; ++h) tot += red[group][h][0];
  const float mu = tot * inv_d;
  float m2 = 0.f;
#pragma unroll
  for (int h = 0; h < W; ++h) {
    const float c = count(h);
    const float dm = (c > 0.f ? red[group][h][0] / c : 0.f) - mu;
    m2 += red[group][h][1] + c * dm * dm;
  }
  const float rs = 1.0f / sqrtf(m2 * inv_d + kEps);
  if (part == 0 && lane == 0) {
    mean[r] = mu;
    rstd[r] = rs;
  }
  if constexpr (fwd_rows_rewiden(V, E)) {
#pragma unroll
    for (int k = 0; k < V; ++k) opaque(xv[k]), opaque(sv[k]), opaque(hv[k]);
  }
  // (late loads: the asm gives the row's modulation pointers a new value
  // here, after the statistics, so the loads below cannot move up)
  const T *srow = scale + mod * D, *hrow = shift + mod * D;
  if constexpr (kLate) asm volatile("" : "+s"(srow), "+s"(hrow));
#pragma unroll
  for (int k = 0; k < V; ++k) {
    if (ok[k]) {
      float o[E];
      if constexpr (kLate) {
        sv[k] = load_vec(srow + (int64_t)jl[k] * E);
        hv[k] = load_vec(hrow + (int64_t)jl[k] * E);
      }
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

// Rows per launch: kMaxGrid workgroups of 4 / W rows.
template <typename T, int V, int W, bool FULL, class Map>
hipError_t fwd_wide_v(int64_t rows, const Map &map, const void *x,
                      const void *scale, const void *shift, void *y,
                      float *mean, float *rstd, int32_t D, hipStream_t s) {
  constexpr int kRows = kBlock / kWave / W;
  constexpr int64_t kRowsPerLaunch = kMaxGrid * kRows;
  for (int64_t first = 0; first < rows; first += kRowsPerLaunch) {
    const int64_t end =
        rows - first < kRowsPerLaunch ? rows : first + kRowsPerLaunch;
    const hipError_t e = launch_kernel(
        fwd_wide_kernel<T, V, W, FULL, Map>, (end - first + kRows - 1) / kRows,
        s, (const T *)x, (const T *)scale, (const T *)shift, (T *)y, mean,
        rstd, D, first, end, map);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}


template <int W, class Map>
hipError_t fwd_wide_dispatch_w(int dtype, int V, int64_t rows, const Map &map,
                               const void *x, const void *scale,
                               const void *shift, void *y, float *mean,
                               float *rstd, int32_t D, hipStream_t stream) {
  const int E = dtype == 1 ? 8 : 4;
  const bool full = (int64_t)V * W * kWave * E == D;
#define ADALN_FWD_WIDE_CASE(V_)                                              \
  if (V == V_) {                                                             \
    if (dtype == 1)                                                          \
      return full ? fwd_wide_v<bf16, V_, W, true>(rows, map, x, scale,       \
                                                  shift, y, mean, rstd, D,   \
                                                  stream)                    \
                  : fwd_wide_v<bf16, V_, W, false>(rows, map, x, scale,      \
                                                   shift, y, mean, rstd, D,  \
                                                   stream);                  \
    return full ? fwd_wide_v<float, V_, W, true>(rows, map, x, scale, shift, \
                                                 y, mean, rstd, D, stream)   \
                : fwd_wide_v<float, V_, W, false>(rows, map, x, scale,       \
                                                  shift, y, mean, rstd, D,   \
                                                  stream);                   \
  }
  if constexpr (W == 2) {
    ADALN_FWD_PAIR_V(ADALN_FWD_WIDE_CASE)
  } else {
    ADALN_FWD_QUAD_V(ADALN_FWD_WIDE_CASE)
  }
#undef ADALN_FWD_WIDE_CASE
  return hipErrorInvalidValue;
}

template <class Map>
hipError_t fwd_wide_dispatch(int dtype, const StreamPlan &plan, int64_t rows,
                             const Map &map, const void *x, const void *scale,
                             const void *shift, void *y, float *mean,
                             float *rstd, int32_t D, hipStream_t stream) {
  if (plan.W == 2)
    return fwd_wide_dispatch_w<2>(dtype, plan.V, rows, map, x, scale, shift,
                                  y, mean, rstd, D, stream);
  if (plan.W == 4)
    return fwd_wide_dispatch_w<4>(dtype, plan.V, rows, map, x, scale, shift,
                                  y, mean, rstd, D, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fwd_wide(int dtype, const StreamPlan &plan, const void *x,
                           const void *scale, const void *shift, void *y,
                           float *mean, float *rstd, int32_t B, int32_t N,
                           int32_t D, hipStream_t stream) {
  return fwd_wide_dispatch(dtype, plan, (int64_t)B * N, BatchRows{N}, x,
                           scale, shift, y, mean, rstd, D, stream);
}

hipError_t launch_fwd_wide_segments(int dtype, const StreamPlan &plan,
                                    const SegMap &map, const void *x,
                                    const void *scale, const void *shift,
                                    void *y, float *mean, float *rstd,
                                    int32_t D, hipStream_t stream) {
  return fwd_wide_dispatch(dtype, plan, map.row_start[map.nseg], map, x,
                           scale, shift, y, mean, rstd, D, stream);
}

}  // namespace adaln
