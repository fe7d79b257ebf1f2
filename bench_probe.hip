// Streaming-bandwidth probes for the benchmark (bench.py), built into
// bench_probe.so beside it; not part of the operator's library.  They run
// the access pattern of the operator's row-stream kernels with no
// arithmetic, to measure what HBM sustains for it on the same buffers:
//
//   kind 0: copy          dst = a           (one read stream, one write)
//   kind 1: read2 write1  dst = a ^ b       (the fused backward's pattern)
//
// Organisation of the row-stream kernels: 256 workgroups of four
// wavefronts, one 10 KiB row per wavefront per step, grid-stride over the
// rows, nontemporal 16-byte loads and stores, every lane one vector per
// instruction.
//
// bench_window_probe walks the rows the way the persistent kernels (the
// backward's) walk a batch of B samples: bps workgroups per sample, grid /
// bps samples in flight, the wavefronts of a sample's workgroups taking rows
// k_in*4 + w, stride 4*bps, from (b * skew) % N rows in (wrapping); with one
// sample and bps = grid = rows / 4 it is the forward's grid of one row per
// wavefront.  Same two kinds, rows of 1 to 10 KiB.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kWave = 64;
constexpr int kProbeV = 10;  // vectors per lane per row: rows of 10 KiB
constexpr int64_t kRow = (int64_t)kProbeV * kWave * 16;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int KIND>
__global__ __launch_bounds__(256) void probe_kernel(
    const u32x4 *__restrict__ a, const u32x4 *__restrict__ b,
    u32x4 *__restrict__ dst, int64_t rows) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  for (int64_t r = (int64_t)blockIdx.x * 4 + wave; r < rows;
       r += (int64_t)gridDim.x * 4) {
    const int64_t base = r * kProbeV * kWave + lane;
    u32x4 va[kProbeV], vb[kProbeV];
#pragma unroll
    for (int k = 0; k < kProbeV; ++k) {
      va[k] = __builtin_nontemporal_load(a + base + k * kWave);
      if (KIND == 1) vb[k] = __builtin_nontemporal_load(b + base + k * kWave);
    }
#pragma unroll
    for (int k = 0; k < kProbeV; ++k) {
      u32x4 o = va[k];
      if (KIND == 1) o ^= vb[k];
      __builtin_nontemporal_store(o, dst + base + k * kWave);
    }
  }
}

template <int KIND, int CV>
__global__ __launch_bounds__(256) void window_probe_kernel(
    const u32x4 *__restrict__ a, const u32x4 *__restrict__ b,
    u32x4 *__restrict__ dst, int B, int N, int bps, int skew) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int groups = gridDim.x / bps;
  const int g = blockIdx.x / bps;
  const int k_in = blockIdx.x % bps;
  if (g >= groups) return;  // workgroups past the last whole group idle
  for (int s = g; s < B; s += groups) {
    const int rot = (int)(((int64_t)s * skew) % N);
    for (int n = k_in * 4 + wave; n < N; n += 4 * bps) {
      const int p = n + rot < N ? n + rot : n + rot - N;
      const int64_t base = ((int64_t)s * N + p) * CV * kWave + lane;
      u32x4 va[CV], vb[CV];
#pragma unroll
      for (int k = 0; k < CV; ++k) {
        va[k] = __builtin_nontemporal_load(a + base + k * kWave);
        if (KIND == 1) vb[k] = __builtin_nontemporal_load(b + base + k * kWave);
      }
#pragma unroll
      for (int k = 0; k < CV; ++k) {
        u32x4 o = va[k];
        if (KIND == 1) o ^= vb[k];
        __builtin_nontemporal_store(o, dst + base + k * kWave);
      }
    }
  }
}

template <int CV>
const void *window_kernel(int kind) {
  return kind == 0 ? (const void *)window_probe_kernel<0, CV>
                   : (const void *)window_probe_kernel<1, CV>;
}

}  // namespace

// Returns 0, -1 for invalid arguments (kind not 0 or 1, a NULL or
// misaligned buffer, bytes not a multiple of 10240), or -5 when the launch
// fails.  a, b, dst: device buffers of `bytes` bytes, 16-byte aligned, not
// overlapping (b unused for kind 0).  Enqueued on `stream`, not waited for.
extern "C" __attribute__((visibility("default"))) int bench_stream_probe(
    int kind, const void *a, const void *b, void *dst, int64_t bytes,
    void *stream) {
  if ((kind != 0 && kind != 1) || bytes < 0 || bytes % kRow != 0) return -1;
  if (bytes == 0) return 0;
  if (a == nullptr || dst == nullptr || (kind == 1 && b == nullptr))
    return -1;
  if ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(dst) |
       reinterpret_cast<uintptr_t>(b)) % 16 != 0)
    return -1;
  int64_t rows = bytes / kRow;
  const u32x4 *pa = static_cast<const u32x4 *>(a);
  const u32x4 *pb = static_cast<const u32x4 *>(b);
  u32x4 *pd = static_cast<u32x4 *>(dst);
  void *args[] = {&pa, &pb, &pd, &rows};
  const void *k = kind == 0 ? (const void *)probe_kernel<0>
                            : (const void *)probe_kernel<1>;
  const hipError_t e = hipLaunchKernel(k, dim3(256), dim3(256), args, 0,
                                       (hipStream_t)stream);
  return e == hipSuccess ? 0 : -5;
}

// The windowed walk over B samples of N rows of row_kib KiB (1 to 10) in
// buffers of B * N * row_kib KiB.  grid workgroups, bps (1 <= bps <= grid)
// per sample, skew >= 0 rows.  Returns 0, -1 for invalid arguments (as for
// bench_stream_probe, plus sizes out of range), or -5 when the launch fails.
extern "C" __attribute__((visibility("default"))) int bench_window_probe(
    int kind, const void *a, const void *b, void *dst, int B, int N,
    int row_kib, int bps, int grid, int skew, void *stream) {
  if ((kind != 0 && kind != 1) || B <= 0 || N <= 0 || row_kib < 1 ||
      row_kib > kProbeV || bps < 1 || grid < bps || grid > 65535 || skew < 0)
    return -1;
  if ((int64_t)B * N > ((int64_t)1 << 40) / 1024) return -1;
  if (a == nullptr || dst == nullptr || (kind == 1 && b == nullptr))
    return -1;
  if ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(dst) |
       reinterpret_cast<uintptr_t>(b)) % 16 != 0)
    return -1;
  const void *k = nullptr;
  switch (row_kib) {
    case 1: k = window_kernel<1>(kind); break;
    case 2: k = window_kernel<2>(kind); break;
    case 3: k = window_kernel<3>(kind); break;
    case 4: k = window_kernel<4>(kind); break;
    case 5: k = window_kernel<5>(kind); break;
    case 6: k = window_kernel<6>(kind); break;
    case 7: k = window_kernel<7>(kind); break;
    case 8: k = window_kernel<8>(kind); break;
    case 9: k = window_kernel<9>(kind); break;
    case 10: k = window_kernel<10>(kind); break;
  }
  const u32x4 *pa = static_cast<const u32x4 *>(a);
  const u32x4 *pb = static_cast<const u32x4 *>(b);
  u32x4 *pd = static_cast<u32x4 *>(dst);
  void *args[] = {&pa, &pb, &pd, &B, &N, &bps, &skew};
  const hipError_t e = hipLaunchKernel(k, dim3(grid), dim3(256), args, 0,
                                       (hipStream_t)stream);
  return e == hipSuccess ? 0 : -5;
}
