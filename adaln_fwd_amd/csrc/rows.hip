// Row kernel of the input gradient dx on its own (adaln_bwd_dx, and the
// backward of rows too wide for the fused kernel): the exact gradient of
// y = xhat * (1 + scale) + shift with respect to x, reusing the mean and rstd
// the forward pass saved.  One token row of D features lives in the
// registers of W wavefronts (V 16-byte vectors per lane); the two row sums
// are reduced inside the wavefront with DPP and across wavefronts in LDS.
#include "common.hpp"
#include "launch.hpp"

namespace adaln {

// Sums of two values over the W wavefronts of a row group, through 8 floats
// of LDS; callers alternate between two such arrays so a barrier always
// separates a read of one from the next write to it.
template <int W>
__device__ __forceinline__ void group_sum2(float &a, float &b, float *red,
                                           int wave, int grp) {
  wave_sum2(a, b);
  if constexpr (W != 1) {
    if (lane_id() == 0) {
      red[wave] = a;
      red[4 + wave] = b;
    }
    __syncthreads();
    float ta = red[grp * W], tb = red[4 + grp * W];
#pragma unroll
    for (int w = 1; w < W; ++w) {
      ta += red[grp * W + w];
      tb += red[4 + grp * W + w];
    }
    a = ta;
    b = tb;
  }
}

template <typename T, int V, int W>
__global__ __launch_bounds__(kBlock) void dx_kernel(
    const T *__restrict__ dy, const T *__restrict__ x,
    const T *__restrict__ scale, const float *__restrict__ mean,
    const float *__restrict__ rstd, T *__restrict__ dx, int32_t rows,
    int32_t N, int32_t D) {
  constexpr int E = Elems<T>::value;
  constexpr int G = 4 / W;
  __shared__ float red[2][8];
  const int lane = lane_id();
  const int wave = wave_id();
  const int grp = wave / W;
  const int wig = wave - grp * W;
  const int nvec = D / E;
  // 64-bit: near rows = 2^31 - 1 the rounding up and the last block's rows
  // would overflow 32 bits
  const int row_blocks = (int)(((int64_t)rows + G - 1) / G);
  const float inv_d = 1.0f / (float)D;
  int parity = 0;

  for (int rb = blockIdx.x; rb < row_blocks; rb += gridDim.x) {
    const int64_t row = (int64_t)rb * G + grp;
    const bool live = row < rows;
    const int64_t off = (int64_t)(live ? row : 0) * D;
    // row < rows <= 2^31 - 1: the sample index in 32-bit arithmetic
    const int64_t moff =
        (int64_t)(live ? (int)((uint32_t)row / (uint32_t)N) : 0) * D;

    // Loads with no predicate (vectors past the row end read its last
    // vector, and are zeroed before their first use) where the registers
    // allow it: measured on MI355X, bf16 [1, 75600, 5120] 471 -> 386 us,
    // [1, 24000, 24576] 753 -> 602 us, f32 [1, 20000, 16384] 871 -> 700 us.
    // bf16 rows of 16 vectors per lane need the predicated form's registers
    // to keep two wavefronts per SIMD ([2, 7000, 32768] 581 against 615 us).
    constexpr bool kClamp = V * E <= 96;
    Vec xv[V], gv[V], sv[V];
    bool ok[V];
#pragma unroll
    for (int k = 0; k < V; ++k) {
      const int j = (k * W + wig) * kWave + lane;
      ok[k] = live && j < nvec;
      if constexpr (kClamp) {
        const int64_t jl = (int64_t)clamp_vec(j, nvec) * E;
        xv[k] = load_stream(x + off + jl);
        gv[k] = load_stream(dy + off + jl);
        sv[k] = load_vec(scale + moff + jl);
      } else {
        xv[k] = ok[k] ? load_stream(x + off + (int64_t)j * E) : vzero();
        gv[k] = ok[k] ? load_stream(dy + off + (int64_t)j * E) : vzero();
      }
    }
    if constexpr (!kClamp) {
#pragma unroll
      for (int k = 0; k < V; ++k) {
        const int j = (k * W + wig) * kWave + lane;
        sv[k] = ok[k] ? load_vec(scale + moff + (int64_t)j * E) : vzero();
      }
    }
    const float mu = live ? mean[row] : 0.f;
    const float r = live ? rstd[row] : 0.f;
    if constexpr (kClamp) {
      mask_tail(xv, ok);
      mask_tail(gv, ok);
      mask_tail(sv, ok);
    }

    // c1 = mean_d(g), c2 = mean_d(g * xhat) with g = dy * (1 + scale)
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
    group_sum2<W>(s1, s2, red[parity], wave, grp);
#pragma unroll
    for (int k = 0; k < V; ++k) {
      opaque(xv[k]);
      opaque(gv[k]);
      opaque(sv[k]);
    }
    parity ^= 1;
    const float c1 = s1 * inv_d;
    const float c2 = s2 * inv_d;

#pragma unroll
    for (int k = 0; k < V; ++k) {
      if (ok[k]) {
        const int64_t c = (int64_t)((k * W + wig) * kWave + lane) * E;
        float o[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float xh = (elem<T>(xv[k], e) - mu) * r;
          const float g = elem<T>(gv[k], e) * (1.0f + elem<T>(sv[k], e));
          o[e] = r * fmaf(-xh, c2, g - c1);
        }
        store_stream(dx + off + c, pack<T>(o));
      }
    }
  }
}

// ------------------------------------------------------------------ dispatch

namespace {

template <typename T, int V, int W>
hipError_t dx_vw(const void *dy, const void *x, const void *scale,
                 const float *mean, const float *rstd, void *dx, int64_t rows,
                 int32_t N, int32_t D, hipStream_t s) {
  constexpr int G = 4 / W;
  return launch_kernel(dx_kernel<T, V, W>, (rows + G - 1) / G, s,
                       (const T *)dy, (const T *)x, (const T *)scale, mean,
                       rstd, (T *)dx, (int32_t)rows, N, D);
}

}  // namespace

#define ADALN_DX_CASE(V_, W_)                                               \
  if (plan.V == V_ && plan.W == W_)                                         \
    return dtype == 1 ? dx_vw<bf16, V_, W_>(dy, x, scale, mean, rstd, dx,   \
                                            rows, N, D, stream)             \
                      : dx_vw<float, V_, W_>(dy, x, scale, mean, rstd, dx,  \
                                             rows, N, D, stream);

hipError_t launch_bwd_dx(int dtype, const RowPlan &plan, const void *dy,
                         const void *x, const void *scale, const float *mean,
                         const float *rstd, void *dx, int64_t rows, int32_t N,
                         int32_t D, hipStream_t stream) {
  ADALN_ROW_PLANS(ADALN_DX_CASE)
  return hipErrorInvalidValue;
}

}  // namespace adaln
