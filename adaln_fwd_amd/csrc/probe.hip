// Streaming-bandwidth probes: the access patterns of the operator's kernels
// with no arithmetic, to measure what HBM sustains for them on this part.
//
//   kind 0: copy          dst = a           (one read stream, one write)
//   kind 1: read2 write1  dst = a ^ b       (the fused backward's pattern)
//
// Same organisation as the row-stream kernels: 256 workgroups of four
// wavefronts, one 10 KiB row per wavefront per step, grid-stride over the
// rows, nontemporal 16-byte loads and stores, every lane one vector per
// instruction.
#include "adaln.h"
#include "common.hpp"
#include "launch.hpp"

namespace adaln {

namespace {

constexpr int kProbeV = 10;  // vectors per lane per row: rows of 10 KiB

template <int KIND>
__global__ __launch_bounds__(kBlock) void probe_kernel(
    const Vec *__restrict__ a, const Vec *__restrict__ b, Vec *__restrict__ dst,
    int64_t rows) {
  const int lane = lane_id();
  const int wave = wave_id();
  for (int64_t r = (int64_t)blockIdx.x * 4 + wave; r < rows;
       r += (int64_t)gridDim.x * 4) {
    const int64_t base = r * kProbeV * kWave + lane;
    Vec va[kProbeV], vb[kProbeV];
#pragma unroll
    for (int k = 0; k < kProbeV; ++k) {
      va[k] = load_stream(a + base + k * kWave);
      if (KIND == 1) vb[k] = load_stream(b + base + k * kWave);
    }
#pragma unroll
    for (int k = 0; k < kProbeV; ++k) {
      Vec o = va[k];
      if (KIND == 1)
#pragma unroll
        for (int i = 0; i < 4; ++i) o.w[i] ^= vb[k].w[i];
      store_stream(dst + base + k * kWave, o);
    }
  }
}

}  // namespace

}  // namespace adaln

using namespace adaln;

extern "C" __attribute__((visibility("default"))) int adaln_stream_probe(
    int kind, const void *a, const void *b, void *dst, int64_t bytes,
    void *stream) {
  constexpr int64_t kRow = (int64_t)kProbeV * kWave * 16;
  if (kind != 0 && kind != 1)
    return fail(ADALN_ERR_INVALID, "probe kind %d is not 0 or 1", kind);
  if (bytes < 0 || bytes % kRow != 0)
    return fail(ADALN_ERR_ALIGN, "probe bytes must be a multiple of %lld",
                (long long)kRow);
  if (bytes == 0) return ok();
  if (a == nullptr || dst == nullptr || (kind == 1 && b == nullptr))
    return fail(ADALN_ERR_INVALID, "probe buffer is NULL");
  if ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(dst) |
       reinterpret_cast<uintptr_t>(b)) % 16 != 0)
    return fail(ADALN_ERR_ALIGN, "probe buffers must be 16-byte aligned");
  const int64_t rows = bytes / kRow;
  const hipError_t e =
      kind == 0
          ? launch_kernel(probe_kernel<0>, kCUs, (hipStream_t)stream,
                          (const Vec *)a, (const Vec *)b, (Vec *)dst, rows)
          : launch_kernel(probe_kernel<1>, kCUs, (hipStream_t)stream,
                          (const Vec *)a, (const Vec *)b, (Vec *)dst, rows);
  if (e != hipSuccess)
    return fail(ADALN_ERR_HIP, "adaln_stream_probe launch: %s",
                hipGetErrorString(e));
  return ok();
}
