// Forward kernels of the fused AdaLN operator (AdaptiveLoad technical
// summary, section 2.B, forward pass): per token row, mean and variance over
// D, then y = xhat * (1 + scale[b]) + shift[b], with x read from HBM once and
// y written once, in a single launch.
//
// fwd_stream_kernel (rows of up to 1024 16-byte vectors): one wavefront per
// row, lane l holding vectors k*64 + l, k < V, in registers; no barrier is
// needed.  A small persistent grid (OCC four-wavefront workgroups per CU) is
// spread over the samples, bps workgroups per sample, and each wavefront
// walks its sample's rows with a stride of 4*bps rows.  All wavefronts that
// are active at a time therefore touch a narrow window of rows that sweeps
// through memory in order: measured on MI355X, that keeps HBM about 15%
// busier than giving each workgroup its own contiguous block of rows.  The
// sample's scale and shift stay in registers.  Mean and variance are
// two-pass over the register-resident row (DPP reductions).
//
// fwd_tile_kernel (wider rows): the W wavefronts of a workgroup share each
// row, lane l of wavefront w holding vectors (k*W + w)*64 + l.  Rows are
// dealt out as in the stream kernel (workgroup k_in of a sample's bps walks
// rows k_in, k_in + bps, ...), with the next row in flight.  Each wavefront
// computes the mean of its own elements and the centred sum of squares
// around it; the W results are combined through LDS with the pairwise update
// of Chan, Golub and LeVeque (1979),
//     M2 = sum_w M2_w + sum_w n_w * (mean_w - mean)^2,
// one barrier per row, keeping the accuracy of a two-pass variance.
//
// All sums run in a fixed order, so results are reproducible bit for bit.
#include "common.hpp"
#include "launch.hpp"

namespace adaln {

template <typename T, int V, bool FULL, int PF, int OCC, class Map>
__global__ __launch_bounds__(kBlock)
__attribute__((amdgpu_waves_per_eu(OCC, OCC))) void fwd_stream_kernel(
    const T *__restrict__ x, const T *__restrict__ scale,
    const T *__restrict__ shift, T *__restrict__ y, float *__restrict__ mean,
    float *__restrict__ rstd, int32_t D, Map map) {
  constexpr int E = Elems<T>::value;
  constexpr int kWaves = kBlock / kWave;
  const int lane = lane_id();
  const int wave = wave_id();
  const int nvec = D / E;
  const float inv_d = 1.0f / (float)D;

  int jv[V];
  bool ok[V];
#pragma unroll
  for (int k = 0; k < V; ++k) {
    jv[k] = k * kWave + lane;
    ok[k] = FULL || jv[k] < nvec;
  }

  // One segment (a sample, or a packed sequence): rows [row0, row0 + N),
  // modulated by vector `mod`; this workgroup is number k_in of bps.
  for_each_segment(map, [&](int64_t row0, int N, int mod, int k_in, int bps,
                            int, int) {
    const int stride = bps * kWaves;
    Vec sv[V], hv[V];
#pragma unroll
    for (int k = 0; k < V; ++k) {
      const int64_t c = (int64_t)mod * D + (int64_t)jv[k] * E;
      sv[k] = ok[k] ? load_vec(scale + c) : vzero();
      hv[k] = ok[k] ? load_vec(shift + c) : vzero();
    }

    auto load_row = [&](Vec (&xv)[V], int n) {
      const int64_t off = (row0 + n) * D;
#pragma unroll
      for (int k = 0; k < V; ++k)
        xv[k] = ok[k] ? load_stream(x + off + (int64_t)jv[k] * E) : vzero();
    };

    auto do_row = [&](Vec (&xv)[V], int n) {
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < V; ++k)
#pragma unroll
        for (int e = 0; e < E; ++e) s += elem<T>(xv[k], e);
      const float mu = wave_sum(s) * inv_d;
#pragma unroll
      for (int k = 0; k < V; ++k) opaque(xv[k]);
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
      const float r = 1.0f / sqrtf(wave_sum(q) * inv_d + kEps);
      if (lane == 0) {
        mean[row0 + n] = mu;
        rstd[row0 + n] = r;
      }
#pragma unroll
      for (int k = 0; k < V; ++k) opaque(xv[k]);
      // Rows of 3 and of 10 or more vectors: widen scale and shift to float
      // again for every row.  Kept widened across the loop they do not fit
      // the register budget of the occupancy these rows run at, and the
      // spills cost more than the conversions (measured: 3-vector bf16 rows
      // 52 -> 32 us for 77 MB).
      if constexpr (V == 3 || V >= 10) {
#pragma unroll
        for (int k = 0; k < V; ++k) opaque(sv[k]), opaque(hv[k]);
      }
      const int64_t off = (row0 + n) * D;
#pragma unroll
      for (int k = 0; k < V; ++k) {
        if (ok[k]) {
          float o[E];
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const float xh = (elem<T>(xv[k], e) - mu) * r;
            o[e] = fmaf(xh, 1.0f + elem<T>(sv[k], e), elem<T>(hv[k], e));
          }
          store_stream(y + off + (int64_t)jv[k] * E, pack<T>(o));
        }
      }
    };

    int n = k_in * kWaves + wave;
    if constexpr (PF == 1) {
      for (; n < N; n += stride) {
        Vec xv[V];
        load_row(xv, n);
        do_row(xv, n);
      }
    } else if (n < N) {
      // the next row of this wavefront is in flight while one is processed;
      // in the loop body every load is unconditional
      Vec xa[V], xb[V];
      load_row(xa, n);
      for (; n + 2 * stride < N; n += 2 * stride) {
        load_row(xb, n + stride);
        do_row(xa, n);
        load_row(xa, n + 2 * stride);
        do_row(xb, n + stride);
      }
      if (n + stride < N) {
        load_row(xb, n + stride);
        do_row(xa, n);
        do_row(xb, n + stride);
      } else {
        do_row(xa, n);
      }
    }
  });
}

// Rows in flight per wavefront of the tile kernel: two, except for the
// 8-vector bfloat16 rows (up to 4096 vectors), whose second row in flight
// does not fit the register budget of two wavefronts per SIMD.
template <typename T, int V>
constexpr int fwd_tile_pf() {
  return (V >= 8 && Elems<T>::value == 8) ? 1 : 2;
}

template <typename T, int V, bool FULL, class Map>
__global__ __launch_bounds__(kMaxRowWaves * kWave)
__attribute__((amdgpu_waves_per_eu(fwd_waves_per_simd(V)))) void fwd_tile_kernel(
    const T *__restrict__ x, const T *__restrict__ scale,
    const T *__restrict__ shift, T *__restrict__ y, float *__restrict__ mean,
    float *__restrict__ rstd, int32_t D, Map map) {
  constexpr int E = Elems<T>::value;
  __shared__ float red[2][3][kMaxRowWaves];  // [parity][sum, m2, count][wave]
  const int lane = lane_id();
  const int wave = wave_id();
  const int W = __builtin_amdgcn_readfirstlane(blockDim.x / kWave);
  const int nvec = D / E;
  const float inv_d = 1.0f / (float)D;

  int jv[V];
  bool ok[V];
  int nvalid = 0;  // vectors this wavefront holds (wave-uniform)
#pragma unroll
  for (int k = 0; k < V; ++k) {
    jv[k] = (k * W + wave) * kWave + lane;
    ok[k] = FULL || jv[k] < nvec;
    const int first = (k * W + wave) * kWave;
    nvalid += FULL ? kWave : max(0, min(kWave, nvec - first));
  }
  const float cnt_w = (float)(nvalid * E);
  int parity = 0;

  for_each_segment(map, [&](int64_t row0, int N, int mod, int k_in, int bps,
                            int, int) {
    Vec sv[V], hv[V];
#pragma unroll
    for (int k = 0; k < V; ++k) {
      const int64_t c = (int64_t)mod * D + (int64_t)jv[k] * E;
      sv[k] = ok[k] ? load_vec(scale + c) : vzero();
      hv[k] = ok[k] ? load_vec(shift + c) : vzero();
    }

    auto load_row = [&](Vec (&xv)[V], int n) {
      const int64_t off = (row0 + n) * D;
#pragma unroll
      for (int k = 0; k < V; ++k)
        xv[k] = ok[k] ? load_stream(x + off + (int64_t)jv[k] * E) : vzero();
    };

    auto do_row = [&](Vec (&xv)[V], int n) {
      // this wavefront's mean and centred sum of squares
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < V; ++k)
#pragma unroll
        for (int e = 0; e < E; ++e) s += elem<T>(xv[k], e);
      const float sum_w = wave_sum(s);
      const float mean_w = cnt_w > 0.f ? sum_w / cnt_w : 0.f;
#pragma unroll
      for (int k = 0; k < V; ++k) opaque(xv[k]);
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
        red[parity][0][wave] = sum_w;
        red[parity][1][wave] = m2_w;
        red[parity][2][wave] = cnt_w;
      }
      __syncthreads();
      float tot = red[parity][0][0];
      for (int w = 1; w < W; ++w) tot += red[parity][0][w];
      const float mu = tot * inv_d;
      float m2 = 0.f;
      for (int w = 0; w < W; ++w) {
        const float cw = red[parity][2][w];
        const float dm = (cw > 0.f ? red[parity][0][w] / cw : 0.f) - mu;
        m2 += red[parity][1][w] + cw * dm * dm;
      }
      parity ^= 1;
      const float r = 1.0f / sqrtf(m2 * inv_d + kEps);
      if (wave == 0 && lane == 0) {
        mean[row0 + n] = mu;
        rstd[row0 + n] = r;
      }

#pragma unroll
      for (int k = 0; k < V; ++k) opaque(xv[k]);
      // as in the stream kernel: re-widen scale and shift per row where
      // keeping them widened would spill
      if constexpr (V >= 4) {
#pragma unroll
        for (int k = 0; k < V; ++k) opaque(sv[k]), opaque(hv[k]);
      }
      const int64_t off = (row0 + n) * D;
#pragma unroll
      for (int k = 0; k < V; ++k) {
        if (ok[k]) {
          float o[E];
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const float xh = (elem<T>(xv[k], e) - mu) * r;
            o[e] = fmaf(xh, 1.0f + elem<T>(sv[k], e), elem<T>(hv[k], e));
          }
          store_stream(y + off + (int64_t)jv[k] * E, pack<T>(o));
        }
      }
    };

    // Steady state: A holds row n and rows n+1, n+2 exist, so every load in
    // the loop body is unconditional; the last one or two rows follow it.
    int n = k_in;
    if constexpr (fwd_tile_pf<T, V>() == 1) {
      for (; n < N; n += bps) {
        Vec xv[V];
        load_row(xv, n);
        do_row(xv, n);
      }
    } else if (n < N) {
      const int stride = bps;
      Vec xa[V], xb[V];
      load_row(xa, n);
      for (; n + 2 * stride < N; n += 2 * stride) {
        load_row(xb, n + stride);
        do_row(xa, n);
        load_row(xa, n + 2 * stride);
        do_row(xb, n + stride);
      }
      if (n + stride < N) {
        load_row(xb, n + stride);
        do_row(xa, n);
        do_row(xb, n + stride);
      } else {
        do_row(xa, n);
      }
    }
  });
}

namespace {

template <typename T, int V, bool FULL, class Map>
hipError_t fwd_tile_v(int64_t grid, int W, const Map &map, const void *x,
                      const void *scale, const void *shift, void *y,
                      float *mean, float *rstd, int32_t D, hipStream_t s) {
  return launch_kernel_threads(fwd_tile_kernel<T, V, FULL, Map>, grid,
                               W * kWave, s, (const T *)x, (const T *)scale,
                               (const T *)shift, (T *)y, mean, rstd, D, map);
}

template <typename T, int V, bool FULL, class Map>
hipError_t fwd_stream_v(int64_t grid, const Map &map, const void *x,
                        const void *scale, const void *shift, void *y,
                        float *mean, float *rstd, int32_t D, hipStream_t s) {
  return launch_kernel(
      fwd_stream_kernel<T, V, FULL, fwd_stream_pf(V), fwd_stream_occ(V), Map>,
      grid, s, (const T *)x, (const T *)scale, (const T *)shift, (T *)y, mean,
      rstd, D, map);
}

}  // namespace

#define ADALN_FWD_STREAM_CASE(V_)                                            \
  if (V == V_) {                                                             \
    if (full)                                                                \
      return dtype == 1 ? fwd_stream_v<bf16, V_, true>(grid, map, x, scale,   \
                                                       shift, y, mean, rstd,  \
                                                       D, stream)             \
                        : fwd_stream_v<float, V_, true>(grid, map, x, scale,  \
                                                        shift, y, mean, rstd, \
                                                        D, stream);           \
    return dtype == 1 ? fwd_stream_v<bf16, V_, false>(grid, map, x, scale,    \
                                                      shift, y, mean, rstd,   \
                                                      D, stream)              \
                      : fwd_stream_v<float, V_, false>(grid, map, x, scale,   \
                                                       shift, y, mean, rstd,  \
                                                       D, stream);            \
  }

namespace {

template <class Map>
hipError_t fwd_stream_dispatch(int dtype, int V, int64_t grid, const Map &map,
                               const void *x, const void *scale,
                               const void *shift, void *y, float *mean,
                               float *rstd, int32_t D, hipStream_t stream) {
  const int E = dtype == 1 ? 8 : 4;
  const bool full = (int64_t)V * kWave * E == D;
  ADALN_STREAM_V(ADALN_FWD_STREAM_CASE)
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fwd_stream(int dtype, const StreamPlan &plan, const void *x,
                             const void *scale, const void *shift, void *y,
                             float *mean, float *rstd, int32_t B, int32_t N,
                             int32_t D, hipStream_t stream) {
  const UniformMap map{B, N, plan.bps, plan.groups, 0};
  return fwd_stream_dispatch(dtype, plan.V, plan.grid, map, x, scale, shift,
                             y, mean, rstd, D, stream);
}

hipError_t launch_fwd_segments(int dtype, int V, const SegMap &map,
                               const void *x, const void *scale,
                               const void *shift, void *y, float *mean,
                               float *rstd, int32_t D, hipStream_t stream) {
  return fwd_stream_dispatch(dtype, V, map.wg_start[map.nseg], map, x, scale,
                             shift, y, mean, rstd, D, stream);
}

#define ADALN_FWD_TILE_CASE(V_)                                             \
  if (V == V_) {                                                            \
    if (full)                                                               \
      return dtype == 1 ? fwd_tile_v<bf16, V_, true>(grid, W, map, x, scale, \
                                                     shift, y, mean, rstd,  \
                                                     D, stream)             \
                        : fwd_tile_v<float, V_, true>(grid, W, map, x,      \
                                                      scale, shift, y,      \
                                                      mean, rstd, D,        \
                                                      stream);              \
    return dtype == 1 ? fwd_tile_v<bf16, V_, false>(grid, W, map, x, scale,  \
                                                    shift, y, mean, rstd, D, \
                                                    stream)                  \
                      : fwd_tile_v<float, V_, false>(grid, W, map, x, scale, \
                                                     shift, y, mean, rstd,  \
                                                     D, stream);            \
  }

namespace {

template <class Map>
hipError_t fwd_tile_dispatch(int dtype, int V, int W, int64_t grid,
                             const Map &map, const void *x, const void *scale,
                             const void *shift, void *y, float *mean,
                             float *rstd, int32_t D, hipStream_t stream) {
  if (W < 1 || W > kMaxRowWaves) return hipErrorInvalidValue;
  const int E = dtype == 1 ? 8 : 4;
  const bool full = (int64_t)V * W * kWave * E == D;
  ADALN_FWD_V(ADALN_FWD_TILE_CASE)
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fwd_tiles(int dtype, const TilePlan &plan, const void *x,
                            const void *scale, const void *shift, void *y,
                            float *mean, float *rstd, int32_t B, int32_t N,
                            int32_t D, hipStream_t stream) {
  const UniformMap map{B, N, plan.bps, plan.groups, 0};
  return fwd_tile_dispatch(dtype, plan.V, plan.W, plan.grid, map, x, scale,
                           shift, y, mean, rstd, D, stream);
}

hipError_t launch_fwd_tiles_segments(int dtype, const TilePlan &plan,
                                     const SegMap &map, const void *x,
                                     const void *scale, const void *shift,
                                     void *y, float *mean, float *rstd,
                                     int32_t D, hipStream_t stream) {
  return fwd_tile_dispatch(dtype, plan.V, plan.W, map.wg_start[map.nseg],
                           map, x, scale, shift, y, mean, rstd, D, stream);
}

}  // namespace adaln
