// Fused backward of the AdaLN operator: dx and the D-tile partial sums of
// dscale/dshift in one pass over x and dy.
//
// The D-tile coalesced reduction of the AdaptiveLoad technical summary
// (section 2.B, backward pass) pins each thread to a feature and accumulates
// down the token rows of a sequence tile.  dx needs every feature of a row
// for its two row sums, so here one workgroup owns an n_tile of token rows of
// one sample and all D features: its W wavefronts each own one d_tile of
// 64*V vectors (lane l holds vectors (k*W + w)*64 + l, k < V), so each
// wavefront is one (d_tile, n_tile) cell of the grid.  Per row the wavefronts
// reduce sum(g) and sum(g*xhat) with DPP, combine through LDS (one barrier),
// write dx, and add dy*xhat and dy into per-lane float32 accumulators that
// stay in registers down the whole tile.  The next row is loaded before the
// current one is reduced.  x and dy are read once instead of twice, which
// cuts the backward pass from five tensor passes to three.
//
// Partials go to the workspace as [B, n_tiles, D] for dscale and for dshift
// and are summed over n_tiles in index order by dmod_finish_kernel.
#include "common.hpp"
#include "launch.hpp"

namespace adaln {

constexpr int kMaxWaves = 8;  // 512 threads

template <typename T, int V>
__global__ __launch_bounds__(kMaxWaves * kWave) void bwd_fused_kernel(
    const T *__restrict__ dy, const T *__restrict__ x,
    const T *__restrict__ scale, const float *__restrict__ mean,
    const float *__restrict__ rstd, T *__restrict__ dx,
    float *__restrict__ part_scale, float *__restrict__ part_shift,
    int32_t N, int32_t D, int32_t n_tile, int32_t n_tiles,
    int32_t total_tiles) {
  constexpr int E = Elems<T>::value;
  __shared__ float red[2][2][kMaxWaves];  // [parity][sum][wave]
  const int lane = lane_id();
  const int wave = wave_id();
  const int W = __builtin_amdgcn_readfirstlane(blockDim.x / kWave);
  const int nvec = D / E;
  const float inv_d = 1.0f / (float)D;

  int jv[V];
  bool ok[V];
#pragma unroll
  for (int k = 0; k < V; ++k) {
    jv[k] = (k * W + wave) * kWave + lane;
    ok[k] = jv[k] < nvec;
  }
  int parity = 0;

  for (int tile = blockIdx.x; tile < total_tiles; tile += gridDim.x) {
    const int b = tile / n_tiles;
    const int t = tile - b * n_tiles;
    const int n0 = t * n_tile;
    const int n1 = min(N, n0 + n_tile);
    const int64_t row0 = (int64_t)b * N;

    // 1 + scale for this sample, held for the whole tile
    Vec sv[V];
#pragma unroll
    for (int k = 0; k < V; ++k)
      sv[k] = ok[k] ? load_vec(scale + (int64_t)b * D + (int64_t)jv[k] * E)
                    : vzero();

    float acc_s[V][E], acc_h[V][E];
#pragma unroll
    for (int k = 0; k < V; ++k)
#pragma unroll
      for (int e = 0; e < E; ++e) acc_s[k][e] = acc_h[k][e] = 0.f;

    // prefetch the first row
    Vec xa[V], ga[V];
    {
      const int64_t off = (row0 + n0) * D;
#pragma unroll
      for (int k = 0; k < V; ++k) {
        xa[k] = ok[k] ? load_stream(x + off + (int64_t)jv[k] * E) : vzero();
        ga[k] = ok[k] ? load_stream(dy + off + (int64_t)jv[k] * E) : vzero();
      }
    }
    float mu = mean[row0 + n0];
    float r = rstd[row0 + n0];

    for (int n = n0; n < n1; ++n) {
      // issue the next row's loads before touching this one
      const bool more = n + 1 < n1;
      const int64_t noff = (row0 + (more ? n + 1 : n)) * D;
      Vec xb[V], gb[V];
#pragma unroll
      for (int k = 0; k < V; ++k) {
        xb[k] = (more && ok[k]) ? load_stream(x + noff + (int64_t)jv[k] * E)
                                : vzero();
        gb[k] = (more && ok[k]) ? load_stream(dy + noff + (int64_t)jv[k] * E)
                                : vzero();
      }
      const float mu_n = more ? mean[row0 + n + 1] : 0.f;
      const float r_n = more ? rstd[row0 + n + 1] : 0.f;

      // row sums of g = dy * (1 + scale) and g * xhat
      float s1 = 0.f, s2 = 0.f;
#pragma unroll
      for (int k = 0; k < V; ++k) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float xh = (elem<T>(xa[k], e) - mu) * r;
          const float g = elem<T>(ga[k], e) * (1.0f + elem<T>(sv[k], e));
          s1 += g;
          s2 = fmaf(g, xh, s2);
        }
      }
      wave_sum2(s1, s2);
      if (lane == 0) {
        red[parity][0][wave] = s1;
        red[parity][1][wave] = s2;
      }
      __syncthreads();
      float t1 = red[parity][0][0], t2 = red[parity][1][0];
      for (int w = 1; w < W; ++w) {
        t1 += red[parity][0][w];
        t2 += red[parity][1][w];
      }
      parity ^= 1;
      const float c1 = t1 * inv_d;
      const float c2 = t2 * inv_d;

#pragma unroll
      for (int k = 0; k < V; ++k) opaque(xa[k]), opaque(ga[k]);

      const int64_t off = (row0 + n) * D;
#pragma unroll
      for (int k = 0; k < V; ++k) {
        if (ok[k]) {
          float o[E];
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const float xh = (elem<T>(xa[k], e) - mu) * r;
            const float gy = elem<T>(ga[k], e);
            const float g = gy * (1.0f + elem<T>(sv[k], e));
            o[e] = r * fmaf(-xh, c2, g - c1);
            acc_s[k][e] = fmaf(gy, xh, acc_s[k][e]);
            acc_h[k][e] += gy;
          }
          store_stream(dx + off + (int64_t)jv[k] * E, pack<T>(o));
        }
      }

#pragma unroll
      for (int k = 0; k < V; ++k) {
        xa[k] = xb[k];
        ga[k] = gb[k];
      }
      mu = mu_n;
      r = r_n;
    }

    const int64_t po = ((int64_t)b * n_tiles + t) * D;
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

namespace {

template <typename T, int V>
hipError_t fused_v(const FusedPlan &plan, const void *dy, const void *x,
                   const void *scale, const float *mean, const float *rstd,
                   void *dx, float *part_scale, float *part_shift, int32_t B,
                   int32_t N, int32_t D, hipStream_t s) {
  const int32_t total = B * plan.n_tiles;
  return launch_kernel_threads(
      bwd_fused_kernel<T, V>, total, plan.W * kWave, s, (const T *)dy,
      (const T *)x, (const T *)scale, mean, rstd, (T *)dx, part_scale,
      part_shift, N, D, (int32_t)plan.n_tile, (int32_t)plan.n_tiles, total);
}

}  // namespace

#define ADALN_FUSED_CASE(V_)                                                 \
  if (plan.V == V_)                                                          \
    return dtype == 1                                                        \
               ? fused_v<bf16, V_>(plan, dy, x, scale, mean, rstd, dx,       \
                                   part_scale, part_shift, B, N, D, stream) \
               : fused_v<float, V_>(plan, dy, x, scale, mean, rstd, dx,      \
                                    part_scale, part_shift, B, N, D, stream);

hipError_t launch_bwd_fused(int dtype, const FusedPlan &plan, const void *dy,
                            const void *x, const void *scale,
                            const float *mean, const float *rstd, void *dx,
                            float *part_scale, float *part_shift, int32_t B,
                            int32_t N, int32_t D, hipStream_t stream) {
  if (plan.W < 1 || plan.W > kMaxWaves) return hipErrorInvalidValue;
  ADALN_FUSED_V(ADALN_FUSED_CASE)
  return hipErrorInvalidValue;
}

}  // namespace adaln
