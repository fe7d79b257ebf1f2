// Fused backward of the AdaLN operator: dx and the D-tile partial sums of
// dscale/dshift in one pass over x and dy, for rows of up to 320 16-byte
// vectors (wider rows: bwd_wide_kernel, then the separate dx and D-tile
// kernels).
//
// The D-tile coalesced reduction of the AdaptiveLoad technical summary
// (section 2.B, backward pass) pins each thread to a feature and accumulates
// down the token rows of a sequence tile, so that every access of a
// wavefront is contiguous along D.  Here each wavefront owns whole rows (lane
// l holds vectors k*64 + l, k < V), which it needs anyway for the two row
// sums of dx, and keeps one float32 accumulator of dy*xhat and one of dy per
// feature it holds: its lanes are pinned to their features for every row it
// visits, and each of its loads covers 1 KiB of contiguous memory.
//
// Grid: a small persistent grid (OCC four-wavefront workgroups per CU) is
// spread over the samples, bps workgroups per sample, and each wavefront
// walks its sample's rows with a stride of 4*bps rows, so the active
// wavefronts sweep a narrow window of memory in order.  The set of rows a
// workgroup visits in one sample is its sequence tile.  With many samples,
// sample b's walk starts (b * skew) % N rows in and wraps around (the
// planner's skew; rot below), so that the samples' windows are not aligned
// with each other in memory.  At the end of a sample the four wavefronts'
// accumulators are added in wavefront order through LDS and written as one
// partial row per (sample, workgroup): the workspace holds [B, bps, D]
// partial sums for dscale and for dshift, which dmod_finish_kernel adds over
// the bps workgroups in index order.  No floating-point atomics anywhere.
#include "common.hpp"
#include "launch.hpp"

namespace adaln {

template <typename T, int V, bool FULL, int PF, int OCC, class Map>
__global__ __launch_bounds__(kBlock)
__attribute__((amdgpu_waves_per_eu(OCC, OCC))) void bwd_stream_kernel(
    const T *__restrict__ dy, const T *__restrict__ x,
    const T *__restrict__ scale, const float *__restrict__ mean,
    const float *__restrict__ rstd, T *__restrict__ dx,
    float *__restrict__ part_scale, float *__restrict__ part_shift,
    int32_t D, Map map) {
  constexpr int E = Elems<T>::value;
  constexpr int kWaves = kBlock / kWave;
  extern __shared__ float stage[];  // the four wavefronts' accumulators
  const int lane = lane_id();
  const int wave = wave_id();
  const int nvec = D / E;
  const float inv_d = 1.0f / (float)D;

  int jv[V], jl[V];  // vector of lane l, and the vector its loads read
  bool ok[V];
#pragma unroll
  for (int k = 0; k < V; ++k) {
    jv[k] = k * kWave + lane;
    ok[k] = FULL || jv[k] < nvec;
    jl[k] = FULL ? jv[k] : clamp_vec(jv[k], nvec);
  }

  // One segment (a sample, or a packed sequence): rows [row0, row0 + N),
  // modulated by vector `mod`, walked from row row0 + rot; this workgroup
  // is number k_in of bps and writes partial row part_row.
  // Workgroup-uniform (barriers below).
  for_each_segment(map, [&](int64_t row0, int N, int mod, int k_in, int bps,
                            int part_row, int rot) {
    // row of the segment that the walk's n-th position stands for
    auto at = [&](int n) -> int64_t {
      const int p = n + rot;
      return row0 + (p >= N ? p - N : p);
    };
    const int stride = bps * kWaves;
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

    auto load_row = [&](Vec (&xv)[V], Vec (&gv)[V], float (&st)[2], int n) {
      st[0] = mean[at(n)];
      st[1] = rstd[at(n)];
      const int64_t off = at(n) * D;
#pragma unroll
      for (int k = 0; k < V; ++k) {
        xv[k] = load_stream(x + off + (int64_t)jl[k] * E);
        gv[k] = load_stream(dy + off + (int64_t)jl[k] * E);
      }
    };

    auto do_row = [&](Vec (&xv)[V], Vec (&gv)[V], const float (&st)[2],
                      int n) {
      if constexpr (!FULL) mask_tail(xv, ok), mask_tail(gv, ok);
      const float mu = st[0];
      const float r = st[1];
      // row sums of g = dy * (1 + scale) and g * xhat
      float s1 = 0.f, s2 = 0.f;
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
      const float c1 = s1 * inv_d;
      const float c2 = s2 * inv_d;
#pragma unroll
      for (int k = 0; k < V; ++k) opaque(xv[k]), opaque(gv[k]);

      const int64_t off = at(n) * D;
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
    };

    // The walk compares n with N - stride rather than n + stride with N, so
    // that no position past N is ever formed: near N = 2^31 - 1 that sum
    // would overflow.
    int n = k_in * kWaves + wave;
    if constexpr (PF == 1) {
      if (n < N) {
        for (;;) {
          Vec xv[V], gv[V];
          float st[2];
          load_row(xv, gv, st, n);
          do_row(xv, gv, st, n);
          if (n >= N - stride) break;
          n += stride;
        }
      }
    } else if (n < N) {
      // the wavefront's next row is in flight while one is processed; in the
      // loop body every load is unconditional
      Vec xa[V], ga[V], xb[V], gb[V];
      float sa[2], sb[2];
      load_row(xa, ga, sa, n);
      for (; n < N - 2 * stride; n += 2 * stride) {
        load_row(xb, gb, sb, n + stride);
        do_row(xa, ga, sa, n);
        load_row(xa, ga, sa, n + 2 * stride);
        do_row(xb, gb, sb, n + stride);
      }
      if (n < N - stride) {
        load_row(xb, gb, sb, n + stride);
        do_row(xa, ga, sa, n);
        do_row(xb, gb, sb, n + stride);
      } else {
        do_row(xa, ga, sa, n);
      }
    }

    // Add the four wavefronts' accumulators in wavefront order and write
    // them as one partial row.
    if constexpr (bwd_stage_all(V, E)) {
      // All four stage theirs ([wave][value][lane]: conflict-free), one
      // barrier, then wavefront w adds and writes the float4 groups g = w,
      // w + 4, ... of the 2*V*E/4 groups (values 4g .. 4g + 3).
      __syncthreads();  // the previous segment's reads of stage are done
#pragma unroll
      for (int k = 0; k < V; ++k)
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int v = wave * V * E + k * E + e;
          stage[(v * 2 + 0) * kWave + lane] = acc_s[k][e];
          stage[(v * 2 + 1) * kWave + lane] = acc_h[k][e];
        }
      __syncthreads();
      constexpr int kGroups = V * E / 4;  // float4 groups per array
      const int64_t po = (int64_t)part_row * D;
#pragma unroll
      for (int gi = 0; gi < (2 * kGroups + kWaves - 1) / kWaves; ++gi) {
        const int g = gi * kWaves + wave;
        if (g < 2 * kGroups) {
          const int a = g / kGroups;         // 0: dscale, 1: dshift
          const int kq = g - a * kGroups;    // k * (E / 4) + q
          const int k = kq / (E / 4);
          if (ok[k]) {
            float v4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int val = kq * 4 + i;    // k * E + e
              float t = stage[((0 * V * E + val) * 2 + a) * kWave + lane];
#pragma unroll
              for (int w = 1; w < kWaves; ++w)
                t += stage[((w * V * E + val) * 2 + a) * kWave + lane];
              v4[i] = t;
            }
            const int q = kq - k * (E / 4);
            const int64_t c = po + (int64_t)jv[k] * E + 4 * q;
            float *dst = a == 0 ? part_scale : part_shift;
            *reinterpret_cast<float4 *>(dst + c) =
                make_float4(v4[0], v4[1], v4[2], v4[3]);
          }
        }
      }
    } else {
      // Add the four wavefronts' accumulators in wavefront order: wavefront w
      // (w = 1, 2, 3) stages its values, wavefront 0 adds them.  Lane-major
      // layout [value][lane] keeps the LDS accesses conflict-free.
#pragma unroll 1
      for (int w = 1; w < kWaves; ++w) {
        __syncthreads();
        if (wave == w) {
#pragma unroll
          for (int k = 0; k < V; ++k)
#pragma unroll
            for (int e = 0; e < E; ++e) {
              stage[((k * E + e) * 2 + 0) * kWave + lane] = acc_s[k][e];
              stage[((k * E + e) * 2 + 1) * kWave + lane] = acc_h[k][e];
            }
        }
        __syncthreads();
        if (wave == 0) {
#pragma unroll
          for (int k = 0; k < V; ++k)
#pragma unroll
            for (int e = 0; e < E; ++e) {
              acc_s[k][e] += stage[((k * E + e) * 2 + 0) * kWave + lane];
              acc_h[k][e] += stage[((k * E + e) * 2 + 1) * kWave + lane];
            }
        }
      }
      if (wave == 0) {
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
    }
  });
}

namespace {

template <typename T, int V, bool FULL, class Map>
hipError_t bwd_stream_v(int64_t grid, const Map &map, const void *dy,
                        const void *x, const void *scale, const float *mean,
                        const float *rstd, void *dx, float *part_scale,
                        float *part_shift, int32_t D, hipStream_t s) {
  constexpr int E = Elems<T>::value;
  const int staged = bwd_stage_all(V, E) ? kBlock / kWave : 1;  // wavefronts
  const size_t lds = (size_t)staged * V * E * 2 * kWave * sizeof(float);
  return launch_kernel_lds(
      bwd_stream_kernel<T, V, FULL, bwd_stream_pf(V), bwd_stream_occ(V), Map>,
      grid, kBlock, lds, s, (const T *)dy, (const T *)x, (const T *)scale,
      mean, rstd, (T *)dx, part_scale, part_shift, D, map);
}

}  // namespace

#define ADALN_BWD_STREAM_CASE(V_)                                             \
  if (V == V_) {                                                              \
    if (full)                                                                 \
      return dtype == 1                                                       \
                 ? bwd_stream_v<bf16, V_, true>(grid, map, dy, x, scale,      \
                                                mean, rstd, dx, part_scale,   \
                                                part_shift, D, stream)        \
                 : bwd_stream_v<float, V_, true>(grid, map, dy, x, scale,     \
                                                 mean, rstd, dx, part_scale,  \
                                                 part_shift, D, stream);      \
    return dtype == 1                                                         \
               ? bwd_stream_v<bf16, V_, false>(grid, map, dy, x, scale, mean, \
                                               rstd, dx, part_scale,          \
                                               part_shift, D, stream)         \
               : bwd_stream_v<float, V_, false>(grid, map, dy, x, scale,      \
                                                mean, rstd, dx, part_scale,   \
                                                part_shift, D, stream);       \
  }

namespace {

template <class Map>
hipError_t bwd_stream_dispatch(int dtype, int V, int64_t grid, const Map &map,
                               const void *dy, const void *x,
                               const void *scale, const float *mean,
                               const float *rstd, void *dx, float *part_scale,
                               float *part_shift, int32_t D,
                               hipStream_t stream) {
  const int E = dtype == 1 ? 8 : 4;
  const bool full = (int64_t)V * kWave * E == D;
  ADALN_BWD_STREAM_V(ADALN_BWD_STREAM_CASE)
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_bwd_fused(int dtype, const StreamPlan &plan, const void *dy,
                            const void *x, const void *scale,
                            const float *mean, const float *rstd, void *dx,
                            float *part_scale, float *part_shift, int32_t B,
                            int32_t N, int32_t D, hipStream_t stream) {
  const UniformMap map{B, N, plan.bps, plan.groups, plan.skew};
  return bwd_stream_dispatch(dtype, plan.V, plan.grid, map, dy, x, scale,
                             mean, rstd, dx, part_scale, part_shift, D,
                             stream);
}

hipError_t launch_bwd_segments(int dtype, int V, const SegMap &map,
                               const void *dy, const void *x,
                               const void *scale, const float *mean,
                               const float *rstd, void *dx, float *part_scale,
                               float *part_shift, int32_t D,
                               hipStream_t stream) {
  return bwd_stream_dispatch(dtype, V, map.wg_start[map.nseg], map, dy, x,
                             scale, mean, rstd, dx, part_scale, part_shift, D,
                             stream);
}

}  // namespace adaln
