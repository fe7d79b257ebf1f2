// Fused backward for rows of 321 to 1280 16-byte vectors (bf16 D of 2568 to
// 10240, f32 D of 1284 to 5120): dx and the D-tile partial sums of
// dscale/dshift in one pass over x and dy, like bwd_stream_kernel, with each
// row split between two wavefronts.
//
// A row held in one wavefront together with its per-lane accumulators (2
// floats per element it owns) takes the whole register file from 640
// vectors up, and outgrows it past that; from 321 vectors up it already
// leaves room for one wavefront per SIMD only, with nothing to cover memory
// latency.  Here the four wavefronts of a workgroup form two pairs; a pair
// shares a row, wavefront h of the pair owning the contiguous vectors
// [h*V*64, (h+1)*V*64) (lane l: vector (h*V + k)*64 + l), so each keeps the
// registers of half the row: two wavefronts per SIMD for rows of up to 640
// vectors, one for wider ones.  The two row sums of dx
// (of g and of g*xhat) are combined through LDS: each wavefront reduces its
// half with DPP, lane 0 stores the two values, one barrier, and both read the
// pair's two halves and add them in half order.  The store area is
// double-buffered by iteration parity, so one barrier per row step
// suffices: a wavefront can reuse a buffer only after every wavefront has
// passed the next barrier, that is after it has read the buffer.
//
// As in the D-tile reduction of the AdaptiveLoad technical summary (section
// 2.B, backward pass), every lane stays pinned to its features for all the
// rows it visits and accumulates dy*xhat and dy in float32.  At the end of a
// segment the two pairs' accumulators (same features, different rows) are
// added in pair order through LDS and written as one partial row per
// (segment, workgroup) -- the workspace layout of bwd_stream_kernel, summed
// by the same finishing kernels.  Fixed-order sums only; no atomics.
#include "common.hpp"
#include "launch.hpp"

namespace adaln {

namespace {

constexpr int kPairs = 2;  // rows a workgroup works on at a time

}  // namespace

template <typename T, int V, bool FULL, class Map>
__global__ __launch_bounds__(kBlock)
__attribute__((amdgpu_waves_per_eu(bwd_wide_occ(V), bwd_wide_occ(V)))) void
bwd_wide_kernel(
    const T *__restrict__ dy, const T *__restrict__ x,
    const T *__restrict__ scale, const float *__restrict__ mean,
    const float *__restrict__ rstd, T *__restrict__ dx,
    float *__restrict__ part_scale, float *__restrict__ part_shift,
    int32_t D, Map map) {
  constexpr int E = Elems<T>::value;
  extern __shared__ float stage[];  // [half][value][lane], one quantity
  __shared__ float sums[2][kPairs][2][2];  // [parity][pair][half][s1, s2]
  const int lane = lane_id();
  const int wave = wave_id();
  const int pair = wave >> 1;
  const int half = wave & 1;
  const int nvec = D / E;
  const float inv_d = 1.0f / (float)D;

  int jv[V];
  bool ok[V];
#pragma unroll
  for (int k = 0; k < V; ++k) {
    jv[k] = (half * V + k) * kWave + lane;
    ok[k] = FULL || jv[k] < nvec;
  }

  int parity = 0;
  // One segment: rows [row0, row0 + N) modulated by vector `mod`, walked
  // from row row0 + rot (the planner keeps rot = 0 for this kernel); this
  // workgroup is number k_in of bps and writes partial row part_row.  Every
  // wavefront of the workgroup runs the same number of loop iterations
  // (barriers below); a pair without a row in the last one only takes part
  // in its barrier.
  for_each_segment(map, [&](int64_t row0, int N, int mod, int k_in, int bps,
                            int part_row, int rot) {
    // row of the segment that the walk's n-th position stands for
    auto at = [&](int n) -> int64_t {
      const int p = n + rot;
      return row0 + (p >= N ? p - N : p);
    };
    const int stride = bps * kPairs;
    Vec sv[V];
#pragma unroll
    for (int k = 0; k < V; ++k)
      sv[k] = ok[k] ? load_vec(scale + (int64_t)mod * D + (int64_t)jv[k] * E)
                    : vzero();

    float acc_s[V][E], acc_h[V][E];
#pragma unroll
    for (int k = 0; k < V; ++k)
#pragma unroll
      for (int e = 0; e < E; ++e) acc_s[k][e] = acc_h[k][e] = 0.f;

    const int first = k_in * kPairs;
    const int iters = first < N ? (N - 1 - first) / stride + 1 : 0;
#pragma unroll 1
    for (int it = 0; it < iters; ++it) {
      const int n = first + pair + it * stride;
      const bool live = n < N;  // uniform across the wavefront
      const int64_t off = at(n) * D;
      Vec xv[V], gv[V];
      float mu = 0.f, r = 0.f, s1 = 0.f, s2 = 0.f;
      if (live) {
        mu = mean[at(n)];
        r = rstd[at(n)];
#pragma unroll
        for (int k = 0; k < V; ++k) {
          xv[k] = ok[k] ? load_stream(x + off + (int64_t)jv[k] * E) : vzero();
          gv[k] = ok[k] ? load_stream(dy + off + (int64_t)jv[k] * E) : vzero();
        }
        // this half's sums of g = dy * (1 + scale) and g * xhat (vectors
        // past the row end hold dy = 0, so g = 0 there)
#pragma unroll
        for (int k = 0; k < V; ++k) {
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const float xh = (elem<T>(xv[k], e) - mu) * r;
            const float g = elem<T>(gv[k], e) * (1.0f + elem<T>(sv[k], e));
            s1 += g;
            s2 = fmaf(g, xh, s2);
          }
        }
        wave_sum2(s1, s2);
      }
      if (lane == 0) {
        sums[parity][pair][half][0] = s1;
        sums[parity][pair][half][1] = s2;
      }
      __syncthreads();
      if (live) {
        const float c1 =
            (sums[parity][pair][0][0] + sums[parity][pair][1][0]) * inv_d;
        const float c2 =
            (sums[parity][pair][0][1] + sums[parity][pair][1][1]) * inv_d;
#pragma unroll
        for (int k = 0; k < V; ++k) opaque(xv[k]), opaque(gv[k]);
#pragma unroll
        for (int k = 0; k < V; ++k) {
          if (ok[k]) {
            float o[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
              const float xh = (elem<T>(xv[k], e) - mu) * r;
              const float gy = elem<T>(gv[k], e);
              const float g = gy * (1.0f + elem<T>(sv[k], e));
              o[e] = r * fmaf(-xh, c2, g - c1);
              acc_s[k][e] = fmaf(gy, xh, acc_s[k][e]);
              acc_h[k][e] += gy;
            }
            store_stream(dx + off + (int64_t)jv[k] * E, pack<T>(o));
          }
        }
      }
      parity ^= 1;
    }

    // Add pair 1's accumulators to pair 0's (same features), one quantity
    // at a time through LDS ([half][value][lane]), then pair 0 writes the
    // partial row, each wavefront its half.  The first barrier keeps the
    // staging area from being overwritten while the previous segment's
    // values are still being read.
    float *st = stage + (size_t)half * V * E * kWave;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      __syncthreads();
      if (pair == 1) {
#pragma unroll
        for (int k = 0; k < V; ++k)
#pragma unroll
          for (int e = 0; e < E; ++e)
            st[(k * E + e) * kWave + lane] = q == 0 ? acc_s[k][e] : acc_h[k][e];
      }
      __syncthreads();
      if (pair == 0) {
#pragma unroll
        for (int k = 0; k < V; ++k)
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const float v = st[(k * E + e) * kWave + lane];
            if (q == 0)
              acc_s[k][e] += v;
            else
              acc_h[k][e] += v;
          }
      }
    }
    if (pair == 0) {
      const int64_t po = (int64_t)part_row * D;
#pragma unroll
      for (int k = 0; k < V; ++k) {
        if (ok[k]) {
          const int64_t c = po + (int64_t)jv[k] * E;
#pragma unroll
          for (int q = 0; q < E / 4; ++q) {
            *reinterpret_cast<float4 *>(part_scale + c + 4 * q) =
                make_float4(acc_s[k][4 * q], acc_s[k][4 * q + 1],
                            acc_s[k][4 * q + 2], acc_s[k][4 * q + 3]);
            *reinterpret_cast<float4 *>(part_shift + c + 4 * q) =
                make_float4(acc_h[k][4 * q], acc_h[k][4 * q + 1],
                            acc_h[k][4 * q + 2], acc_h[k][4 * q + 3]);
          }
        }
      }
    }
  });
}

namespace {

template <typename T, int V, bool FULL, class Map>
hipError_t bwd_wide_v(int64_t grid, const Map &map, const void *dy,
                      const void *x, const void *scale, const float *mean,
                      const float *rstd, void *dx, float *part_scale,
                      float *part_shift, int32_t D, hipStream_t s) {
  constexpr int E = Elems<T>::value;
  const size_t lds = (size_t)kWideWaves * V * E * kWave * sizeof(float);
  return launch_kernel_lds(bwd_wide_kernel<T, V, FULL, Map>, grid, kBlock,
                           lds, s, (const T *)dy, (const T *)x,
                           (const T *)scale, mean, rstd, (T *)dx, part_scale,
                           part_shift, D, map);
}

template <class Map>
hipError_t bwd_wide_dispatch(int dtype, int V, int64_t grid, const Map &map,
                             const void *dy, const void *x, const void *scale,
                             const float *mean, const float *rstd, void *dx,
                             float *part_scale, float *part_shift, int32_t D,
                             hipStream_t stream) {
  const int E = dtype == 1 ? 8 : 4;
  const bool full = (int64_t)V * kWideWaves * kWave * E == D;
#define ADALN_BWD_WIDE_CASE(V_)                                               \
  if (V == V_) {                                                              \
    if (dtype == 1)                                                           \
      return full ? bwd_wide_v<bf16, V_, true>(grid, map, dy, x, scale, mean, \
                                               rstd, dx, part_scale,          \
                                               part_shift, D, stream)         \
                  : bwd_wide_v<bf16, V_, false>(grid, map, dy, x, scale,      \
                                                mean, rstd, dx, part_scale,   \
                                                part_shift, D, stream);       \
    return full ? bwd_wide_v<float, V_, true>(grid, map, dy, x, scale, mean,  \
                                              rstd, dx, part_scale,           \
                                              part_shift, D, stream)          \
                : bwd_wide_v<float, V_, false>(grid, map, dy, x, scale, mean, \
                                               rstd, dx, part_scale,          \
                                               part_shift, D, stream);        \
  }
  ADALN_BWD_WIDE_V(ADALN_BWD_WIDE_CASE)
#undef ADALN_BWD_WIDE_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_bwd_wide(int dtype, const StreamPlan &plan, const void *dy,
                           const void *x, const void *scale,
                           const float *mean, const float *rstd, void *dx,
                           float *part_scale, float *part_shift, int32_t B,
                           int32_t N, int32_t D, hipStream_t stream) {
  const UniformMap map{B, N, plan.bps, plan.groups, plan.skew};
  return bwd_wide_dispatch(dtype, plan.V, plan.grid, map, dy, x, scale, mean,
                           rstd, dx, part_scale, part_shift, D, stream);
}

hipError_t launch_bwd_wide_segments(int dtype, int V, const SegMap &map,
                                    const void *dy, const void *x,
                                    const void *scale, const float *mean,
                                    const float *rstd, void *dx,
                                    float *part_scale, float *part_shift,
                                    int32_t D, hipStream_t stream) {
  return bwd_wide_dispatch(dtype, V, map.wg_start[map.nseg], map, dy, x,
                           scale, mean, rstd, dx, part_scale, part_shift, D,
                           stream);
}

}  // namespace adaln
