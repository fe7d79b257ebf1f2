// Fused backward for rows of 321 to 4096 16-byte vectors (bf16 D of 2568 to
// 32768, f32 D of 1284 to 16384): dx and the D-tile partial sums of
// dscale/dshift in one pass over x and dy, like bwd_stream_kernel, with each
// row split between W = 2, 4 or 8 wavefronts.
//
// A row held in one wavefront together with its per-lane accumulators (2
// floats per element it owns) takes the whole register file from 640
// vectors up, and outgrows it past that; from 321 vectors up it already
// leaves room for one wavefront per SIMD only, with nothing to cover memory
// latency.  Here the four wavefronts of a workgroup form 4 / W row groups
// (two pairs, or one quad); wavefront h of a group owns the contiguous
// vectors [h*V*64, (h+1)*V*64) of the group's row (lane l: vector
// (h*V + k)*64 + l), so each keeps the registers of 1/W of the row: pairs
// take rows of up to 1280 vectors (two wavefronts per SIMD up to 640), quads
// up to 2560.  Past that, a 512-thread workgroup of eight wavefronts (two per
// SIMD) works on one row at a time, each wavefront an eighth of it, up to
// 4096 vectors.  The two row sums of dx (of g and of g*xhat) are combined
// through LDS: each wavefront reduces its part with DPP, lane 0 stores the
// two values, one barrier, and every wavefront of the group reads the W
// parts and adds them in part order.  The store area is double-buffered by
// iteration parity, so one barrier per row step suffices: a wavefront can
// reuse a buffer only after every wavefront has passed the next barrier,
// that is after it has read the buffer.
//
// As in the D-tile reduction of the AdaptiveLoad technical summary (section
// 2.B, backward pass), every lane stays pinned to its features for all the
// rows it visits and accumulates dy*xhat and dy in float32.  At the end of a
// segment the pairs' accumulators (same features, different rows) are added
// in pair order through LDS -- a quad or an eight-wavefront group owns all
// of its workgroup's rows and needs no such step -- and written as one
// partial row per (segment, workgroup): the workspace layout of
// bwd_stream_kernel, summed by the same finishing kernels.  Fixed-order
// sums only; no atomics.
//
// Two choices are made per row width, by measurement (launch.hpp): PF, the
// rows in flight per wavefront (a second one where it fits beside the
// accumulators), and SPLIT, the loop form at one row in flight (the loads as
// one step and the arithmetic as the next, or both in one branch).  All
// forms do the same arithmetic in the same order.
#include "common.hpp"
#include "launch.hpp"

namespace adaln {

template <typename T, int V, int W, int PF, bool SPLIT, bool FULL, class Map>
__global__ __launch_bounds__(bwd_wide_block(W))
__attribute__((amdgpu_waves_per_eu(bwd_wide_occ(V, W),
                                   bwd_wide_occ(V, W)))) void
bwd_wide_kernel(
    const T *__restrict__ dy, const T *__restrict__ x,
    const T *__restrict__ scale, const float *__restrict__ mean,
    const float *__restrict__ rstd, T *__restrict__ dx,
    float *__restrict__ part_scale, float *__restrict__ part_shift,
    int32_t D, Map map) {
  static_assert(W == 2 || W == 4 || W == 8,
                "a row takes two, four or eight wavefronts");
  constexpr int E = Elems<T>::value;
  constexpr int kRows = bwd_wide_block(W) / kWave / W;  // rows at a time
  extern __shared__ float stage[];  // [part][value][lane], one quantity
  __shared__ float sums[2][kRows][W][2];  // [parity][group][part][s1, s2]
  const int lane = lane_id();
  const int wave = wave_id();
  const int group = wave / W;  // row group of this wavefront
  const int part = wave % W;   // its part of the group's row
  const int nvec = D / E;
  const float inv_d = 1.0f / (float)D;

  int jv[V], jl[V];  // vector of lane l, and the vector its loads read
  bool ok[V];
#pragma unroll
  for (int k = 0; k < V; ++k) {
    jv[k] = (part * V + k) * kWave + lane;
    ok[k] = FULL || jv[k] < nvec;
    jl[k] = FULL ? jv[k] : clamp_vec(jv[k], nvec);
  }
  // Where registers are short, the indices are derived again in each row
  // from a base that an empty asm makes new there, so they are not held
  // across the row loop.
  constexpr bool kIdxRegs = bwd_wide_index_regs(V, W, E);
  int vbase = part * V * kWave + lane;
  auto JV = [&](int k) -> int {
    if constexpr (kIdxRegs) return jv[k];
    else return vbase + k * kWave;
  };
  auto OK = [&](int k) -> bool {
    if constexpr (kIdxRegs) return ok[k];
    else return FULL || vbase + k * kWave < nvec;
  };
  auto JL = [&](int k) -> int {
    if constexpr (kIdxRegs) return jl[k];
    else return FULL ? JV(k) : clamp_vec(JV(k), nvec);
  };
  auto fresh = [&]() {
    if constexpr (!kIdxRegs) asm volatile("" : "+v"(vbase));
  };
  // zero the vectors past the row's end
  auto mask_row = [&](Vec (&xv)[V], Vec (&gv)[V]) {
    if constexpr (!FULL && kIdxRegs) {
      mask_tail(xv, ok), mask_tail(gv, ok);
    } else if constexpr (!FULL) {
      bool okr[V];
#pragma unroll
      for (int k = 0; k < V; ++k) okr[k] = OK(k);
      mask_tail(xv, okr), mask_tail(gv, okr);
    }
  };

  int parity = 0;
  // One segment: rows [row0, row0 + N) modulated by vector `mod`, walked
  // from row row0 + rot (the planner keeps rot = 0 for this kernel); this
  // workgroup is number k_in of bps and writes partial row part_row.  Every
  // wavefront of the workgroup runs the same number of loop iterations
  // (barriers below); a row group without a row in the last one only takes
  // part in its barrier.
  for_each_segment(map, [&](int64_t row0, int N, int mod, int k_in, int bps,
                            int part_row, int rot) {
    // row of the segment that the walk's n-th position stands for
    auto at = [&](int n) -> int64_t {
      const int p = n + rot;
      return row0 + (p >= N ? p - N : p);
    };
    const int stride = bps * kRows;
    // The segment's scale: held in registers for the whole segment, or, where
    // the accumulators leave no room for it, read again (from L2) at each use.
    // The empty asm makes the address new at every use, so the compiler
    // cannot hoist those loads out of the row loop into registers.
    constexpr bool kScaleRegs = bwd_wide_scale_regs(V, W, E);
    Vec sv[kScaleRegs ? V : 1];
    if constexpr (kScaleRegs) {
#pragma unroll
      for (int k = 0; k < V; ++k)
        sv[k] = OK(k) ? load_vec(scale + (int64_t)mod * D + (int64_t)JV(k) * E)
                      : vzero();
    }
    auto scale_vec = [&](int k) -> Vec {
      if constexpr (kScaleRegs) {
        return sv[k];
      } else {
        const T *p = scale + (int64_t)mod * D;
        asm volatile("" : "+s"(p));
        return OK(k) ? load_vec(p + (int64_t)JV(k) * E) : vzero();
      }
    };

    float acc_s[V][E], acc_h[V][E];
#pragma unroll
    for (int k = 0; k < V; ++k)
#pragma unroll
      for (int e = 0; e < E; ++e) acc_s[k][e] = acc_h[k][e] = 0.f;

    // the next row of this row group is in flight while one is processed
    // where the registers allow it (PF == 2); load_row skips rows past the
    // segment's end, do_row computes nothing for them but still takes part
    // in the barrier
    auto load_row = [&](Vec (&xv)[V], Vec (&gv)[V], float (&st)[2], int n) {
      if (n < N) {
        st[0] = mean[at(n)];
        st[1] = rstd[at(n)];
        const int64_t off = at(n) * D;
        fresh();
#pragma unroll
        for (int k = 0; k < V; ++k) {
          xv[k] = load_stream(x + off + (int64_t)JL(k) * E);
          gv[k] = load_stream(dy + off + (int64_t)JL(k) * E);
        }
      }
    };

    auto do_row = [&](Vec (&xv)[V], Vec (&gv)[V], const float (&st)[2],
                      int n) {
      const bool live = n < N;  // uniform across the wavefront
      const float mu = st[0];
      const float r = st[1];
      float s1 = 0.f, s2 = 0.f;
      if (live) {
        fresh();
        mask_row(xv, gv);
        // this part's sums of g = dy * (1 + scale) and g * xhat (vectors
        // past the row end hold dy = 0, so g = 0 there)
#pragma unroll
        for (int k = 0; k < V; ++k) {
          const Vec sk = scale_vec(k);
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const float xh = (elem<T>(xv[k], e) - mu) * r;
            const float g = elem<T>(gv[k], e) * (1.0f + elem<T>(sk, e));
            s1 += g;
            s2 = fmaf(g, xh, s2);
          }
        }
        wave_sum2(s1, s2);
      }
      if (lane == 0) {
        sums[parity][group][part][0] = s1;
        sums[parity][group][part][1] = s2;
      }
      __syncthreads();
      if (live) {
        float t1 = sums[parity][group][0][0];
        float t2 = sums[parity][group][0][1];
#pragma unroll
        for (int h = 1; h < W; ++h) {
          t1 += sums[parity][group][h][0];
          t2 += sums[parity][group][h][1];
        }
        const float c1 = t1 * inv_d;
        const float c2 = t2 * inv_d;
#pragma unroll
        for (int k = 0; k < V; ++k) opaque(xv[k]), opaque(gv[k]);
        fresh();
        const int64_t off = at(n) * D;
#pragma unroll
        for (int k = 0; k < V; ++k) {
          if (OK(k)) {
            const Vec sk = scale_vec(k);
            float o[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
              const float xh = (elem<T>(xv[k], e) - mu) * r;
              const float gy = elem<T>(gv[k], e);
              const float g = gy * (1.0f + elem<T>(sk, e));
              o[e] = r * fmaf(-xh, c2, g - c1);
              acc_s[k][e] = fmaf(gy, xh, acc_s[k][e]);
              acc_h[k][e] += gy;
            }
            store_stream(dx + off + (int64_t)JV(k) * E, pack<T>(o));
          }
        }
      }
      parity ^= 1;
    };

    // every wavefront of the workgroup runs `iters` row steps
    const int first = k_in * kRows + group;
    int iters = k_in * kRows < N ? (N - 1 - k_in * kRows) / stride + 1 : 0;
    // The XCD-weighted walk (kXcdM > 0, launch.hpp): rounds of kXcdM regular
    // steps of the plain walk (positions j, j + stride, ... for walker
    // j = k_in * kRows + group), then one extra step for the walkers of
    // workgroups with an even block index, which take the positions after
    // the regular ones in walker order.  A round covers kXcdM * stride + Wf
    // positions, Wf the number of such walkers of the segment; a segment's
    // workgroups start at block index blockIdx.x - k_in, so those with
    // k_in of that parity are the even ones.  A row group's position is
    // its workgroup's first row group's plus `group` in both kinds of step,
    // so the workgroup's row groups step together.
    constexpr int kXcdM = std::is_same<Map, UniformMap>::value
                              ? bwd_wide_xcd_m(V, W, E, FULL)
                              : 0;  // packed layouts keep the plain walk
    const int q0 = (int)((blockIdx.x - (unsigned)k_in) & 1u);
    const bool even_xcd = (blockIdx.x & 1u) == 0u;
    const int64_t j0 = (int64_t)k_in * kRows;
    const int64_t rank0 = (int64_t)((k_in - q0) / 2) * kRows;
    const int64_t round_len =
        (int64_t)kXcdM * stride +
        (int64_t)(q0 == 0 ? (bps + 1) / 2 : bps / 2) * kRows;
    const int steps = kXcdM + (even_xcd ? 1 : 0);  // per round
    if constexpr (kXcdM > 0) {
      // steps whose first row group's position lies in the segment
      const int64_t t = (int64_t)N / round_len;
      const int64_t rem = (int64_t)N - t * round_len;
      int64_t cnt = t * steps;
      if (rem > j0) cnt += min((int64_t)kXcdM, (rem - j0 - 1) / stride + 1);
      if (even_xcd && (int64_t)kXcdM * stride + rank0 < rem) cnt += 1;
      iters = (int)cnt;
    }
    // the walk position of step `it` for this row group (N past the end)
    auto pos = [&](int it) -> int {
      if constexpr (kXcdM == 0) {
        return first + it * stride;
      } else {
        const int t = it / steps, r = it - t * steps;
        const int64_t p =
            (int64_t)t * round_len +
            (r < kXcdM ? (int64_t)r * stride + j0
                       : (int64_t)kXcdM * stride + rank0) +
            group;
        return p < N ? (int)p : N;
      }
    };
    if constexpr (PF == 1 && SPLIT) {
#pragma unroll 1
      for (int it = 0; it < iters; ++it) {
        Vec xv[V], gv[V];
        float st[2] = {0.f, 0.f};
        load_row(xv, gv, st, pos(it));
        do_row(xv, gv, st, pos(it));
      }
    } else if constexpr (PF == 1) {
      // the same steps with the loads and the first pass in one branch
      // (the compiler schedules the two forms differently; which is faster
      // depends on the row width)
#pragma unroll 1
      for (int it = 0; it < iters; ++it) {
        const int n = pos(it);
        const bool live = n < N;  // uniform across the wavefront
        const int64_t off = at(n) * D;
        Vec xv[V], gv[V];
        float mu = 0.f, r = 0.f, s1 = 0.f, s2 = 0.f;
        if (live) {
          mu = mean[at(n)];
          r = rstd[at(n)];
          fresh();
#pragma unroll
          for (int k = 0; k < V; ++k) {
            xv[k] = load_stream(x + off + (int64_t)JL(k) * E);
            gv[k] = load_stream(dy + off + (int64_t)JL(k) * E);
          }
          mask_row(xv, gv);
#pragma unroll
          for (int k = 0; k < V; ++k) {
            const Vec sk = scale_vec(k);
#pragma unroll
            for (int e = 0; e < E; ++e) {
              const float xh = (elem<T>(xv[k], e) - mu) * r;
              const float g = elem<T>(gv[k], e) * (1.0f + elem<T>(sk, e));
              s1 += g;
              s2 = fmaf(g, xh, s2);
            }
          }
          wave_sum2(s1, s2);
        }
        if (lane == 0) {
          sums[parity][group][part][0] = s1;
          sums[parity][group][part][1] = s2;
        }
        __syncthreads();
        if (live) {
          float t1 = sums[parity][group][0][0];
          float t2 = sums[parity][group][0][1];
#pragma unroll
          for (int h = 1; h < W; ++h) {
            t1 += sums[parity][group][h][0];
            t2 += sums[parity][group][h][1];
          }
          const float c1 = t1 * inv_d;
          const float c2 = t2 * inv_d;
#pragma unroll
          for (int k = 0; k < V; ++k) opaque(xv[k]), opaque(gv[k]);
          fresh();
#pragma unroll
          for (int k = 0; k < V; ++k) {
            if (OK(k)) {
              const Vec sk = scale_vec(k);
              float o[E];
#pragma unroll
              for (int e = 0; e < E; ++e) {
                const float xh = (elem<T>(xv[k], e) - mu) * r;
                const float gy = elem<T>(gv[k], e);
                const float g = gy * (1.0f + elem<T>(sk, e));
                o[e] = r * fmaf(-xh, c2, g - c1);
                acc_s[k][e] = fmaf(gy, xh, acc_s[k][e]);
                acc_h[k][e] += gy;
              }
              store_stream(dx + off + (int64_t)JV(k) * E, pack<T>(o));
            }
          }
        }
        parity ^= 1;
      }
    } else if (iters > 0) {
      Vec xa[V], ga[V], xb[V], gb[V];
      float sa[2] = {0.f, 0.f}, sb[2] = {0.f, 0.f};
      int it = 0;
      load_row(xa, ga, sa, pos(0));
#pragma unroll 1
      for (; it + 2 < iters; it += 2) {
        load_row(xb, gb, sb, pos(it + 1));
        do_row(xa, ga, sa, pos(it));
        load_row(xa, ga, sa, pos(it + 2));
        do_row(xb, gb, sb, pos(it + 1));
      }
      if (it + 1 < iters) {
        load_row(xb, gb, sb, pos(it + 1));
        do_row(xa, ga, sa, pos(it));
        do_row(xb, gb, sb, pos(it + 1));
      } else {
        do_row(xa, ga, sa, pos(it));
      }
    }

    // Pairs: add pair 1's accumulators to pair 0's (same features), one
    // quantity at a time through LDS ([part][value][lane]), then pair 0
    // writes the partial row, each wavefront its half.  The first barrier
    // keeps the staging area from being overwritten while the previous
    // segment's values are still being read.  A quad or eight-wavefront
    // group is the workgroup's only row group and writes its parts directly.
    if constexpr (kRows == 2) {
      float *st = stage + (size_t)part * V * E * kWave;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        __syncthreads();
        if (group == 1) {
#pragma unroll
          for (int k = 0; k < V; ++k)
#pragma unroll
            for (int e = 0; e < E; ++e)
              st[(k * E + e) * kWave + lane] =
                  q == 0 ? acc_s[k][e] : acc_h[k][e];
        }
        __syncthreads();
        if (group == 0) {
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
    }
    if (group == 0) {
      const int64_t po = (int64_t)part_row * D;
#pragma unroll
      for (int k = 0; k < V; ++k) {
        if (OK(k)) {
          const int64_t c = po + (int64_t)JV(k) * E;
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

template <typename T, int V, int W, bool FULL, class Map>
hipError_t bwd_wide_v(int64_t grid, const Map &map, const void *dy,
                      const void *x, const void *scale, const float *mean,
                      const float *rstd, void *dx, float *part_scale,
                      float *part_shift, int32_t D, hipStream_t s) {
  constexpr int E = Elems<T>::value;
  // staging of the pairs' end-of-segment sum: W parts of V*E floats per lane
  constexpr int kThreads = bwd_wide_block(W);
  const size_t lds =
      kThreads / kWave / W == 2 ? (size_t)W * V * E * kWave * sizeof(float)
                                : 0;
  return launch_kernel_lds(bwd_wide_kernel<T, V, W, bwd_wide_pf(V, W, E, FULL),
                                           bwd_wide_split(V, E), FULL, Map>,
                           grid, kThreads,
                           lds, s, (const T *)dy, (const T *)x,
                           (const T *)scale, mean, rstd, (T *)dx, part_scale,
                           part_shift, D, map);
}

template <int W, class Map>
hipError_t bwd_wide_dispatch_w(int dtype, int V, int64_t grid, const Map &map,
                               const void *dy, const void *x,
                               const void *scale, const float *mean,
                               const float *rstd, void *dx, float *part_scale,
                               float *part_shift, int32_t D,
                               hipStream_t stream) {
  const int E = dtype == 1 ? 8 : 4;
  const bool full = (int64_t)V * W * kWave * E == D;
#define ADALN_BWD_WIDE_CASE(V_)                                               \
  if (V == V_) {                                                              \
    if (dtype == 1)                                                           \
      return full ? bwd_wide_v<bf16, V_, W, true>(grid, map, dy, x, scale,    \
                                                  mean, rstd, dx, part_scale, \
                                                  part_shift, D, stream)      \
                  : bwd_wide_v<bf16, V_, W, false>(grid, map, dy, x, scale,   \
                                                   mean, rstd, dx,            \
                                                   part_scale, part_shift, D, \
                                                   stream);                   \
    return full ? bwd_wide_v<float, V_, W, true>(grid, map, dy, x, scale,     \
                                                 mean, rstd, dx, part_scale,  \
                                                 part_shift, D, stream)       \
                : bwd_wide_v<float, V_, W, false>(grid, map, dy, x, scale,    \
                                                  mean, rstd, dx, part_scale, \
                                                  part_shift, D, stream);     \
  }
  if constexpr (W == 2) {
    ADALN_BWD_PAIR_V(ADALN_BWD_WIDE_CASE)
  } else if constexpr (W == 4) {
    ADALN_BWD_QUAD_V(ADALN_BWD_WIDE_CASE)
  } else {
    ADALN_BWD_OCT_V(ADALN_BWD_WIDE_CASE)
  }
#undef ADALN_BWD_WIDE_CASE
  return hipErrorInvalidValue;
}

template <class Map>
hipError_t bwd_wide_dispatch(int dtype, int V, int W, int64_t grid,
                             const Map &map, const void *dy, const void *x,
                             const void *scale, const float *mean,
                             const float *rstd, void *dx, float *part_scale,
                             float *part_shift, int32_t D,
                             hipStream_t stream) {
  if (W == 2)
    return bwd_wide_dispatch_w<2>(dtype, V, grid, map, dy, x, scale, mean,
                                  rstd, dx, part_scale, part_shift, D, stream);
  if (W == 4)
    return bwd_wide_dispatch_w<4>(dtype, V, grid, map, dy, x, scale, mean,
                                  rstd, dx, part_scale, part_shift, D, stream);
  if (W == 8)
    return bwd_wide_dispatch_w<8>(dtype, V, grid, map, dy, x, scale, mean,
                                  rstd, dx, part_scale, part_shift, D, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_bwd_wide(int dtype, const StreamPlan &plan, const void *dy,
                           const void *x, const void *scale,
                           const float *mean, const float *rstd, void *dx,
                           float *part_scale, float *part_shift, int32_t B,
                           int32_t N, int32_t D, hipStream_t stream) {
  const UniformMap map{B, N, plan.bps, plan.groups, plan.skew};
  return bwd_wide_dispatch(dtype, plan.V, plan.W, plan.grid, map, dy, x,
                           scale, mean, rstd, dx, part_scale, part_shift, D,
                           stream);
}

hipError_t launch_bwd_wide_segments(int dtype, const StreamPlan &plan,
                                    const SegMap &map, const void *dy,
                                    const void *x, const void *scale,
                                    const float *mean, const float *rstd,
                                    void *dx, float *part_scale,
                                    float *part_shift, int32_t D,
                                    hipStream_t stream) {
  return bwd_wide_dispatch(dtype, plan.V, plan.W, map.wg_start[map.nseg], map,
                           dy, x, scale, mean, rstd, dx, part_scale,
                           part_shift, D, stream);
}

}  // namespace adaln
