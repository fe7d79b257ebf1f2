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
// the group's row (lane l: vector (h*V + k)*64 + l) and walks the sample's
// rows with the stream kernels' sample stride.  Each wavefront reduces its
// part with DPP to a sum and a centred sum of squares around the part's own
// mean; lane 0 stores the two values, one barrier, and every wavefront of
// the group combines the W parts in part order with the pairwise update of
// Chan, Golub and LeVeque (1979),
//     mean = sum_h S_h / D,  M2 = sum_h (M2_h + n_h * (S_h / n_h - mean)^2),
// which keeps the accuracy of a two-pass variance.  The store area is
// double-buffered by iteration parity, so one barrier per row step suffices.
// Where the registers allow it the next row is in flight while one is
// processed.  All sums run in a fixed order: results are reproducible bit
// for bit.
//
// Unlike fwd_rows_kernel this kernel keeps a persistent grid at one
// wavefront per SIMD.  A grid of one row per row group with no occupancy
// imposed measured mixed on MI355X (bf16, in one process on the same
// buffers): 1 x 16384 x 12288 150 -> 144 us, but 16 x 1560 x 10240 197 ->
// 258 us, 4 x 4096 x 16384 194 -> 205 us, 1 x 8192 x 32768 226 -> 239 us.
// One row per four-wavefront workgroup for every wide row (5 to 16 vectors
// per lane) was 3-12% slower on all of them.
#include "common.hpp"
#include "launch.hpp"

namespace adaln {

template <typename T, int V, int W, int PF, bool FULL, class Map>
__global__ __launch_bounds__(kBlock)
__attribute__((amdgpu_waves_per_eu(fwd_wide_occ(V), fwd_wide_occ(V)))) void
fwd_wide_kernel(const T *__restrict__ x, const T *__restrict__ scale,
                const T *__restrict__ shift, T *__restrict__ y,
                float *__restrict__ mean, float *__restrict__ rstd,
                int32_t D, Map map) {
  static_assert(W == 2 || W == 4, "a row takes two or four wavefronts");
  constexpr int E = Elems<T>::value;
  constexpr int kRows = kBlock / kWave / W;  // rows a workgroup works on
  __shared__ float red[2][kRows][W][2];  // [parity][group][part][sum, m2]
  const int lane = lane_id();
  const int wave = wave_id();
  const int group = wave / W;  // row group (pair or quad) of this wavefront
  const int part = wave % W;   // its part of the group's row
  const int nvec = D / E;
  const float inv_d = 1.0f / (float)D;

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
  const float cnt_w = count(part);
  int parity = 0;

  // One segment: rows [row0, row0 + N) modulated by vector `mod`; this
  // workgroup is number k_in of bps.  Every wavefront of the workgroup runs
  // the same number of row steps (barriers below); a row group without a
  // row in the last one only takes part in its barrier.
  for_each_segment(map, [&](int64_t row0, int N, int mod, int k_in, int bps,
                            int, int) {
    const int stride = bps * kRows;
    Vec sv[V], hv[V];
#pragma unroll
    for (int k = 0; k < V; ++k) {
      const int64_t c = (int64_t)mod * D + (int64_t)jv[k] * E;
      sv[k] = ok[k] ? load_vec(scale + c) : vzero();
      hv[k] = ok[k] ? load_vec(shift + c) : vzero();
    }

    auto load_row = [&](Vec (&xv)[V], int n) {
      if (n < N) {
        const int64_t off = (row0 + n) * D;
#pragma unroll
        for (int k = 0; k < V; ++k)
          xv[k] = load_stream(x + off + (int64_t)jl[k] * E);
      }
    };

    auto do_row = [&](Vec (&xv)[V], int n) {
      const bool live = n < N;  // uniform across the wavefront
      float sum_w = 0.f, m2_w = 0.f;
      if (live) {
        if constexpr (!FULL) mask_tail(xv, ok);
        // this part's sum, and its centred sum of squares around its mean
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < V; ++k)
#pragma unroll
          for (int e = 0; e < E; ++e) s += elem<T>(xv[k], e);
        sum_w = wave_sum(s);
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
        m2_w = wave_sum(q);
      }
      if (lane == 0) {
        red[parity][group][part][0] = sum_w;
        red[parity][group][part][1] = m2_w;
      }
      __syncthreads();
      if (live) {
        float tot = red[parity][group][0][0];
#pragma unroll
        for (int h = 1; h < W; ++h) tot += red[parity][group][h][0];
        const float mu = tot * inv_d;
        float m2 = 0.f;
#pragma unroll
        for (int h = 0; h < W; ++h) {
          const float c = count(h);
          const float dm = (c > 0.f ? red[parity][group][h][0] / c : 0.f) - mu;
          m2 += red[parity][group][h][1] + c * dm * dm;
        }
        const float r = 1.0f / sqrtf(m2 * inv_d + kEps);
        if (part == 0 && lane == 0) {
          mean[row0 + n] = mu;
          rstd[row0 + n] = r;
        }
#pragma unroll
        for (int k = 0; k < V; ++k) opaque(xv[k]);
        // bf16 rows of 12 and 16 vectors per lane: widen scale and shift to
        // float again for every row; kept widened they would spill
        if constexpr (fwd_wide_rewiden(V, E)) {
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
      }
      parity ^= 1;
    };

    // every wavefront of the workgroup runs `iters` row steps
    const int first = k_in * kRows + group;
    const int iters =
        k_in * kRows < N ? (N - 1 - k_in * kRows) / stride + 1 : 0;
    if constexpr (PF == 1) {
#pragma unroll 1
      for (int it = 0; it < iters; ++it) {
        Vec xv[V];
        load_row(xv, first + it * stride);
        do_row(xv, first + it * stride);
      }
    } else if (iters > 0) {
      Vec xa[V], xb[V];
      int it = 0;
      load_row(xa, first);
#pragma unroll 1
      for (; it + 2 < iters; it += 2) {
        load_row(xb, first + (it + 1) * stride);
        do_row(xa, first + it * stride);
        load_row(xa, first + (it + 2) * stride);
        do_row(xb, first + (it + 1) * stride);
      }
      if (it + 1 < iters) {
        load_row(xb, first + (it + 1) * stride);
        do_row(xa, first + it * stride);
        do_row(xb, first + (it + 1) * stride);
      } else {
        do_row(xa, first + it * stride);
      }
    }
  });
}

namespace {

template <typename T, int V, int W, bool FULL, class Map>
hipError_t fwd_wide_v(int64_t grid, const Map &map, const void *x,
                      const void *scale, const void *shift, void *y,
                      float *mean, float *rstd, int32_t D, hipStream_t s) {
  return launch_kernel(fwd_wide_kernel<T, V, W, fwd_wide_pf(V), FULL, Map>,
                       grid, s, (const T *)x, (const T *)scale,
                       (const T *)shift, (T *)y, mean, rstd, D, map);
}

template <int W, class Map>
hipError_t fwd_wide_dispatch_w(int dtype, int V, int64_t grid, const Map &map,
                               const void *x, const void *scale,
                               const void *shift, void *y, float *mean,
                               float *rstd, int32_t D, hipStream_t stream) {
  const int E = dtype == 1 ? 8 : 4;
  const bool full = (int64_t)V * W * kWave * E == D;
#define ADALN_FWD_WIDE_CASE(V_)                                              \
  if (V == V_) {                                                             \
    if (dtype == 1)                                                          \
      return full ? fwd_wide_v<bf16, V_, W, true>(grid, map, x, scale,       \
                                                  shift, y, mean, rstd, D,   \
                                                  stream)                    \
                  : fwd_wide_v<bf16, V_, W, false>(grid, map, x, scale,      \
                                                   shift, y, mean, rstd, D,  \
                                                   stream);                  \
    return full ? fwd_wide_v<float, V_, W, true>(grid, map, x, scale, shift, \
                                                 y, mean, rstd, D, stream)   \
                : fwd_wide_v<float, V_, W, false>(grid, map, x, scale,       \
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
hipError_t fwd_wide_dispatch(int dtype, const StreamPlan &plan, int64_t grid,
                             const Map &map, const void *x, const void *scale,
                             const void *shift, void *y, float *mean,
                             float *rstd, int32_t D, hipStream_t stream) {
  if (plan.W == 2)
    return fwd_wide_dispatch_w<2>(dtype, plan.V, grid, map, x, scale, shift,
                                  y, mean, rstd, D, stream);
  if (plan.W == 4)
    return fwd_wide_dispatch_w<4>(dtype, plan.V, grid, map, x, scale, shift,
                                  y, mean, rstd, D, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fwd_wide(int dtype, const StreamPlan &plan, const void *x,
                           const void *scale, const void *shift, void *y,
                           float *mean, float *rstd, int32_t B, int32_t N,
                           int32_t D, hipStream_t stream) {
  const UniformMap map{B, N, plan.bps, plan.groups, 0};
  return fwd_wide_dispatch(dtype, plan, plan.grid, map, x, scale, shift, y,
                           mean, rstd, D, stream);
}

hipError_t launch_fwd_wide_segments(int dtype, const StreamPlan &plan,
                                    const SegMap &map, const void *x,
                                    const void *scale, const void *shift,
                                    void *y, float *mean, float *rstd,
                                    int32_t D, hipStream_t stream) {
  return fwd_wide_dispatch(dtype, plan, map.wg_start[map.nseg], map, x, scale,
                           shift, y, mean, rstd, D, stream);
}

}  // namespace adaln
