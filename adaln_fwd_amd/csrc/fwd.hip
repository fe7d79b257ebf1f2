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
// Wider rows: fwd_wide_kernel (fwd_wide.hip).
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

  int jv[V], jl[V];  // vector of lane l, and the vector its load reads
  bool ok[V];
#pragma unroll
  for (int k = 0; k < V; ++k) {
    jv[k] = k * kWave + lane;
    ok[k] = FULL || jv[k] < nvec;
    jl[k] = FULL ? jv[k] : clamp_vec(jv[k], nvec);
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
        xv[k] = load_stream(x + off + (int64_t)jl[k] * E);
    };

    auto do_row = [&](Vec (&xv)[V], int n) {
      if constexpr (!FULL) mask_tail(xv, ok);
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

namespace {

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

}  // namespace adaln
