// Modulation gradients of the fused AdaLN operator through the D-tile
// coalesced reduction (AdaptiveLoad technical summary, section 2.B, backward
// pass): dscale[b,d] = sum_n dy * xhat and dshift[b,d] = sum_n dy.
//
// Reducing along N row by row would walk memory with a stride of D.  Instead
// the grid is cut into (d_tile, n_tile) pieces (times the batch): each lane is
// pinned to the 16 bytes of features it owns and accumulates down the token
// rows of its n_tile, so every load of a wavefront covers 1 KiB of contiguous
// memory.  The four wavefronts of a workgroup take interleaved rows of the
// same n_tile and combine through LDS; each workgroup writes one float32
// partial per feature, and a second kernel sums the partials of the n_tiles
// in index order.  No floating-point atomics: the result is reproducible bit
// for bit.
#include "common.hpp"
#include "launch.hpp"

namespace adaln {

constexpr int kRowsInFlight = 4;  // rows each wavefront loads before using

template <typename T>
__global__ __launch_bounds__(kBlock) void dmod_partial_kernel(
    const T *__restrict__ dy, const T *__restrict__ x,
    const float *__restrict__ mean, const float *__restrict__ rstd,
    float *__restrict__ part_scale, float *__restrict__ part_shift,
    int32_t N, int32_t D, int32_t d_tiles, int32_t n_tile, int32_t n_tiles,
    int64_t total_tiles) {
  constexpr int E = Elems<T>::value;
  constexpr int U = kRowsInFlight;
  constexpr int kWaves = kBlock / kWave;
  __shared__ float stage[kWaves - 1][2 * E][kWave];
  const int lane = lane_id();
  const int wave = wave_id();
  const int nvec = D / E;

  for (int64_t tile = blockIdx.x; tile < total_tiles; tile += gridDim.x) {
    const int dt = (int)(tile % d_tiles);
    const int64_t rest = tile / d_tiles;
    const int t = (int)(rest % n_tiles);
    const int b = (int)(rest / n_tiles);
    const int j = dt * kWave + lane;  // this lane's vector of the row
    const bool ok = j < nvec;
    // No position past the tile end is formed: near N = 2^31 - 1 it would
    // overflow 32 bits.  steps: walk positions of this wavefront in the tile.
    const int n0 = t * n_tile;
    const int n1 = (int)((int64_t)n0 + n_tile < N ? (int64_t)n0 + n_tile : N);
    constexpr int kStep = kWaves * U;
    const int steps = n1 - n0 > wave ? (n1 - n0 - wave - 1) / kStep + 1 : 0;
    const int64_t row0 = (int64_t)b * N;

    float acc_s[E], acc_h[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc_s[e] = acc_h[e] = 0.f;

    for (int i = 0; i < steps; ++i) {
      const int n = n0 + wave + i * kStep;
      Vec xv[U], gv[U];
      float mu[U], r[U];
      bool in[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // no predicate on the loads: rows past the tile and vectors past the
        // row end read a valid address, and are zeroed before their use
        const bool live = u * kWaves < n1 - n;
        const int nn = live ? n + u * kWaves : n0;
        in[u] = live && ok;
        const int64_t off =
            (row0 + (live ? nn : n0)) * D + (int64_t)clamp_vec(j, nvec) * E;
        xv[u] = load_stream(x + off);
        gv[u] = load_stream(dy + off);
        mu[u] = live ? mean[row0 + nn] : 0.f;
        r[u] = live ? rstd[row0 + nn] : 0.f;
      }
      mask_tail(xv, in);
      mask_tail(gv, in);
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float g = elem<T>(gv[u], e);
          const float xh = (elem<T>(xv[u], e) - mu[u]) * r[u];
          acc_s[e] = fmaf(g, xh, acc_s[e]);
          acc_h[e] += g;
        }
      }
    }

    if (wave > 0) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        stage[wave - 1][e][lane] = acc_s[e];
        stage[wave - 1][E + e][lane] = acc_h[e];
      }
    }
    __syncthreads();
    if (wave == 0 && ok) {
#pragma unroll
      for (int w = 0; w < kWaves - 1; ++w) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          acc_s[e] += stage[w][e][lane];
          acc_h[e] += stage[w][E + e][lane];
        }
      }
      const int64_t po = ((int64_t)b * n_tiles + t) * D + (int64_t)j * E;
#pragma unroll
      for (int q = 0; q < E / 4; ++q) {
        *reinterpret_cast<float4 *>(part_scale + po + 4 * q) =
            make_float4(acc_s[4 * q], acc_s[4 * q + 1], acc_s[4 * q + 2],
                        acc_s[4 * q + 3]);
        *reinterpret_cast<float4 *>(part_shift + po + 4 * q) =
            make_float4(acc_h[4 * q], acc_h[4 * q + 1], acc_h[4 * q + 2],
                        acc_h[4 * q + 3]);
      }
    }
    __syncthreads();  // `stage` is reused by the next tile
  }
}

// Waves per workgroup (at most) of the finishing kernels.
constexpr int kFinishWaves = 16;

// log2 of the wavefronts per column block that sum `rows` partial rows at
// most `batch` rows each (at most 16 wavefronts).
static int finish_wpc_log2(int64_t rows, int batch) {
  int l = 0;
  while (l < 4 && rows > (int64_t)batch << l) ++l;
  return l;
}

// dscale[b, d] = sum over t = 0 .. n_tiles-1 of part_scale[b, t, d] (and the
// same for dshift).  The partials are 1-25 MB, so the kernel's time is the
// issue rate of the CUs it runs on: it is spread over as many CUs as the
// shape allows.
//
// A column block is F consecutive features (F = 64, 32 or 16) of one sample.
// A wavefront splits into R = 64 / F lane groups: lane l reads feature
// l % F and its group g = l / F, so one load instruction covers R partial
// rows of the block (R segments of 4F contiguous bytes).  The host picks F
// so that the blocks cover the CUs (64 for 16 samples of 1536 features: 384
// blocks; 32 for one sample of 5120: 160; 16 for one sample of 1536: 96).
// wpc wavefronts (a power of two, at most 16) share a block and cut the
// tiles into wpc contiguous slices; a workgroup holds cpb blocks (wpc * cpb
// <= 16 wavefronts).
//
// Order of the sums, fixed by (n_tiles, F, wpc): in slice j, group g adds
// the tiles t0 + g, t0 + g + R, ... in increasing order (up to kFinishBatch
// loads per array in flight); the R group sums are added in group order
// within the wavefront, and the slice sums in slice order through LDS.  No
// atomics: the result is reproducible bit for bit.  With n_tiles == 0 the
// outputs are zero.
constexpr int kFinishBatch = 8;

// Workgroups are dealt to the 8 XCDs of the part round robin (workgroup i to
// XCD i % 8), and each XCD has its own L2.  This maps workgroup i to a
// logical block so that each XCD takes a contiguous run of blocks: column
// blocks that share a 128-byte line then meet in the same L2.  A bijection of
// [0, grid): the last grid % 8 workgroups keep their own index.
__device__ __forceinline__ int64_t xcd_block(int64_t id, int64_t grid) {
  constexpr int64_t kXcds = 8;
  const int64_t per = grid / kXcds;
  return id < per * kXcds ? (id % kXcds) * per + id / kXcds : id;
}


// First logical block of the calling workgroup.  Only blocks narrower than
// 64 features, which share lines with a neighbour, are remapped: a 64-feature
// block owns whole 256-byte segments, and in the identity order (neighbouring
// blocks on neighbouring XCDs, reading the same rows at once) the packed
// finish ran ~1 us faster (measured on MI355X inside a step, 7.8 against
// 8.7 us for an 11-sequence pack).
template <int F>
__device__ __forceinline__ int64_t first_block() {
  if constexpr (F == 64)
    return blockIdx.x;
  else
    return xcd_block(blockIdx.x, gridDim.x);
}

template <int F>
__global__ __launch_bounds__(kFinishWaves * kWave) void dmod_finish_kernel(
    const float *__restrict__ part_scale, const float *__restrict__ part_shift,
    float *__restrict__ dscale, float *__restrict__ dshift, int32_t D,
    int32_t n_tiles, int32_t col_blocks, int32_t wpc_log2, int32_t cpb,
    int64_t total_cols) {
  constexpr int R = kWave / F;
  __shared__ float stage[kFinishWaves][2][F];
  const int lane = lane_id();
  const int wave = wave_id();
  const int f = lane % F;
  const int g = lane / F;
  const int wpc = 1 << wpc_log2;
  const int slice = wave & (wpc - 1);
  const int t0 = (int)((int64_t)slice * n_tiles / wpc);
  const int t1 = (int)((int64_t)(slice + 1) * n_tiles / wpc);

  for (int64_t blk = first_block<F>(); blk * cpb < total_cols;
       blk += gridDim.x) {
    const int64_t col = blk * cpb + (wave >> wpc_log2);  // (b, column block)
    const bool live = col < total_cols;
    const int cb = live ? (int)(col % col_blocks) : 0;
    const int b = live ? (int)(col / col_blocks) : 0;
    const int c = cb * F + f;
    const bool ok = live && c < D;
    const int64_t base = (int64_t)b * n_tiles * D + c;
    float as = 0.f, ah = 0.f;
    for (int t = t0 + g; t < t1; t += R * kFinishBatch) {
      float vs[kFinishBatch], vh[kFinishBatch];
#pragma unroll
      for (int i = 0; i < kFinishBatch; ++i) {
        const int row = t + i * R;
        const bool in = ok && row < t1;
        vs[i] = in ? part_scale[base + (int64_t)row * D] : 0.f;
        vh[i] = in ? part_shift[base + (int64_t)row * D] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < kFinishBatch; ++i) {
        as += vs[i];
        ah += vh[i];
      }
    }
    // the R lane groups' sums, in group order (lanes of group 0 keep them)
    if constexpr (R > 1) {
      float ts = as, th = ah;
#pragma unroll
      for (int q = 1; q < R; ++q) {
        ts += __shfl(as, lane + q * F);
        th += __shfl(ah, lane + q * F);
      }
      as = ts;
      ah = th;
    }
    if (slice > 0 && g == 0) {
      stage[wave][0][f] = as;
      stage[wave][1][f] = ah;
    }
    __syncthreads();
    if (slice == 0 && g == 0 && ok) {
      for (int w = 1; w < wpc; ++w) {
        as += stage[wave + w][0][f];
        ah += stage[wave + w][1][f];
      }
      dscale[(int64_t)b * D + c] = as;
      dshift[(int64_t)b * D + c] = ah;
    }
    __syncthreads();
  }
}

// Segment variant: dscale[m, d] = sum over the segments s with mod[s] == m,
// in index order, of the partial rows of their workgroups
// [wg_start[s], wg_start[s+1]).  Column blocks, lane groups, slices and
// workgroups as in dmod_finish_kernel (blocks of F features of one
// modulation vector m).  Order: slice j, group g adds, segment by segment in
// index order, the rows wg_start[s] + j + g*wpc, then every R*wpc-th row
// after it, in increasing order (up to kFinishBatch loads per array in
// flight); the group sums are added in group order, the slice sums in slice
// order.
template <int F>
__global__ __launch_bounds__(kFinishWaves * kWave) void finish_segments_kernel(
    const float *__restrict__ part_scale, const float *__restrict__ part_shift,
    float *__restrict__ dscale, float *__restrict__ dshift, int32_t D,
    int32_t col_blocks, int32_t wpc_log2, int32_t cpb, int64_t total_cols,
    SegMap map) {
  constexpr int R = kWave / F;
  __shared__ float stage[kFinishWaves][2][F];
  const int lane = lane_id();
  const int wave = wave_id();
  const int f = lane % F;
  const int g = lane / F;
  const int wpc = 1 << wpc_log2;
  const int slice = wave & (wpc - 1);
  const int step = wpc * R;  // rows between a group's consecutive rows

  for (int64_t blk = first_block<F>(); blk * cpb < total_cols;
       blk += gridDim.x) {
    const int64_t col = blk * cpb + (wave >> wpc_log2);  // (m, column block)
    const bool live = col < total_cols;
    const int cb = live ? (int)(col % col_blocks) : 0;
    const int m = live ? (int)(col / col_blocks) : -1;
    const int c = cb * F + f;
    const bool ok = live && c < D;
    float as = 0.f, ah = 0.f;
    for (int s = 0; s < map.nseg; ++s) {
      if (map.mod[s] != m) continue;
      const int end = map.wg_start[s + 1];
      for (int w0 = map.wg_start[s] + slice + g * wpc; w0 < end;
           w0 += step * kFinishBatch) {
        float vs[kFinishBatch], vh[kFinishBatch];
#pragma unroll
        for (int i = 0; i < kFinishBatch; ++i) {
          const int w = w0 + i * step;
          const bool in = ok && w < end;
          vs[i] = in ? part_scale[(int64_t)w * D + c] : 0.f;
          vh[i] = in ? part_shift[(int64_t)w * D + c] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < kFinishBatch; ++i) {
          as += vs[i];
          ah += vh[i];
        }
      }
    }
    if constexpr (R > 1) {
      float ts = as, th = ah;
#pragma unroll
      for (int q = 1; q < R; ++q) {
        ts += __shfl(as, lane + q * F);
        th += __shfl(ah, lane + q * F);
      }
      as = ts;
      ah = th;
    }
    if (slice > 0 && g == 0) {
      stage[wave][0][f] = as;
      stage[wave][1][f] = ah;
    }
    __syncthreads();
    if (slice == 0 && g == 0 && ok) {
      for (int w = 1; w < wpc; ++w) {
        as += stage[wave + w][0][f];
        ah += stage[wave + w][1][f];
      }
      dscale[(int64_t)m * D + c] = as;
      dshift[(int64_t)m * D + c] = ah;
    }
    __syncthreads();
  }
}

FinishPlan finish_plan(int64_t vectors, int32_t D, int64_t rows) {
  // Column block width: 64 features when that gives every CU a block; else
  // 32 when that still covers half the CUs (16-feature blocks would then
  // put two workgroups on some CUs and split every 128-byte line between
  // two blocks); else 16.  Measured on MI355X inside a step, against 64
  // features and up to 16 wavefronts per workgroup: 16 x 1536 features,
  // 30 partial rows 5.6 -> 4.0 us; 1 x 1536, 512 rows 5.9 -> 4.8 us;
  // 1 x 5120, 511 rows unchanged (6.5 us).
  constexpr int64_t kTargetCols = 256;
  FinishPlan p;
  p.F = 64;
  if (vectors * ((D + 63) / 64) < kTargetCols)
    p.F = vectors * ((D + 31) / 32) >= kTargetCols / 2 ? 32 : 16;
  const int R = kWave / p.F;
  p.wpc = 1 << finish_wpc_log2(rows, R * kFinishBatch);
  p.col_blocks = (D + p.F - 1) / p.F;
  p.total_cols = (int64_t)p.col_blocks * vectors;
  // column blocks per workgroup: as many as keep 256 workgroups or more
  int64_t cpb = p.total_cols / kTargetCols;
  if (cpb > kFinishWaves / p.wpc) cpb = kFinishWaves / p.wpc;
  if (cpb < 1) cpb = 1;
  p.cpb = (int)cpb;
  p.threads = p.wpc * p.cpb * kWave;
  p.blocks = (p.total_cols + cpb - 1) / cpb;
  return p;
}

static int32_t log2_of(int v) {
  int32_t l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

hipError_t launch_finish_segments(const float *part_scale,
                                  const float *part_shift, float *dscale,
                                  float *dshift, const SegMap &map,
                                  int32_t nmod, int32_t D,
                                  hipStream_t stream) {
  // the most partial rows any modulation vector sums
  int64_t most = 0;
  for (int32_t m = 0; m < nmod; ++m) {
    int64_t rows = 0;
    for (int s = 0; s < map.nseg; ++s)
      if (map.mod[s] == m) rows += map.wg_start[s + 1] - map.wg_start[s];
    most = rows > most ? rows : most;
  }
  const FinishPlan sh = finish_plan(nmod, D, most);
  auto go = [&](auto kernel) {
    return launch_kernel_threads(kernel, sh.blocks, sh.threads, stream,
                                 part_scale, part_shift, dscale, dshift, D,
                                 sh.col_blocks, log2_of(sh.wpc),
                                 (int32_t)sh.cpb, sh.total_cols, map);
  };
  return sh.F == 64 ? go(finish_segments_kernel<64>)
                    : sh.F == 32 ? go(finish_segments_kernel<32>)
                                 : go(finish_segments_kernel<16>);
}

hipError_t launch_dmod_partial(int dtype, const DmodPlan &plan,
                               const void *dy, const void *x,
                               const float *mean, const float *rstd,
                               float *part_scale, float *part_shift,
                               int32_t B, int32_t N, int32_t D,
                               hipStream_t stream) {
  const int64_t total_tiles = (int64_t)plan.d_tiles * plan.n_tiles * B;
  if (dtype == 1)
    return launch_kernel(dmod_partial_kernel<bf16>, total_tiles, stream,
                         (const bf16 *)dy, (const bf16 *)x, mean, rstd,
                         part_scale, part_shift, N, D, (int32_t)plan.d_tiles,
                         (int32_t)plan.n_tile, (int32_t)plan.n_tiles,
                         total_tiles);
  return launch_kernel(dmod_partial_kernel<float>, total_tiles, stream,
                       (const float *)dy, (const float *)x, mean, rstd,
                       part_scale, part_shift, N, D, (int32_t)plan.d_tiles,
                       (int32_t)plan.n_tile, (int32_t)plan.n_tiles,
                       total_tiles);
}

hipError_t launch_dmod_finish(const float *part_scale,
                              const float *part_shift, float *dscale,
                              float *dshift, int32_t B, int32_t D,
                              int32_t n_tiles, hipStream_t stream) {
  const FinishPlan sh = finish_plan(B, D, n_tiles);
  auto go = [&](auto kernel) {
    return launch_kernel_threads(kernel, sh.blocks, sh.threads, stream,
                                 part_scale, part_shift, dscale, dshift, D,
                                 n_tiles, sh.col_blocks, log2_of(sh.wpc),
                                 (int32_t)sh.cpb, sh.total_cols);
  };
  return sh.F == 64 ? go(dmod_finish_kernel<64>)
                    : sh.F == 32 ? go(dmod_finish_kernel<32>)
                                 : go(dmod_finish_kernel<16>);
}

}  // namespace adaln
