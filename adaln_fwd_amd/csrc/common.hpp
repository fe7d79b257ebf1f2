// Device helpers shared by the AdaLN kernels (gfx950, wave64).
//
// Storage types: float (4 per 16-byte vector) and bfloat16 (8 per vector).
// Every global access of a token row is one 16-byte vector per lane, so a
// wavefront moves 1 KiB of contiguous memory per instruction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace adaln {

constexpr int kWave = 64;
constexpr int kBlock = 256;  // threads per workgroup for every kernel
constexpr float kEps = 1e-6f;

// bfloat16 storage tag; values are handled as float in registers.
struct bf16 {
  uint16_t bits;
};

template <typename T>
struct Elems;
template <>
struct Elems<float> {
  static constexpr int value = 4;
};
template <>
struct Elems<bf16> {
  static constexpr int value = 8;
};

// 16 bytes of raw storage.
struct alignas(16) Vec {
  uint32_t w[4];
};

__device__ __forceinline__ Vec vzero() {
  Vec v;
  v.w[0] = v.w[1] = v.w[2] = v.w[3] = 0u;
  return v;
}

__device__ __forceinline__ Vec load_vec(const void *p) {
  const uint4 u = *reinterpret_cast<const uint4 *>(p);
  Vec v;
  v.w[0] = u.x;
  v.w[1] = u.y;
  v.w[2] = u.z;
  v.w[3] = u.w;
  return v;
}

__device__ __forceinline__ void store_vec(void *p, const Vec &v) {
  uint4 u;
  u.x = v.w[0];
  u.y = v.w[1];
  u.z = v.w[2];
  u.w = v.w[3];
  *reinterpret_cast<uint4 *>(p) = u;
}

// Streaming access for the [B, N, D] activations, which each kernel touches
// exactly once: the nontemporal hint (the `nt` bit of global_load/store)
// keeps them from displacing reused data in the caches.  Measured on MI355X
// it also raises the sustained rate of read-then-write streams by roughly
// 10% over default-policy accesses.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ Vec load_stream(const void *p) {
  const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  Vec v;
  v.w[0] = u.x;
  v.w[1] = u.y;
  v.w[2] = u.z;
  v.w[3] = u.w;
  return v;
}

__device__ __forceinline__ void store_stream(void *p, const Vec &v) {
  const u32x4 u = {v.w[0], v.w[1], v.w[2], v.w[3]};
  __builtin_nontemporal_store(u, reinterpret_cast<u32x4 *>(p));
}

// Rows whose width is not a whole number of wavefront vectors: lane l's
// vector j may lie past the row end (j >= nvec).  Its load reads the row's
// last vector instead (a valid address, data already being fetched) with no
// predicate, and mask_tail zeroes it at its first use.  A predicated load
// (`ok ? load : 0`) made the compiler wait for all outstanding memory
// traffic right after it, which took away the next row's prefetch.
__device__ __forceinline__ int clamp_vec(int j, int nvec) {
  return j < nvec ? j : nvec - 1;
}

template <int V>
__device__ __forceinline__ void mask_tail(Vec (&v)[V], const bool (&ok)[V]) {
#pragma unroll
  for (int k = 0; k < V; ++k)
    if (!ok[k]) v[k] = vzero();
}

// Make the compiler treat the vector's registers as rewritten here, so later
// uses re-derive float values from the packed registers instead of keeping
// every widened value alive across a reduction (which would double or triple
// the register footprint of a row).  Emits no instruction.
__device__ __forceinline__ void opaque(Vec &v) {
  asm("" : "+v"(v.w[0]), "+v"(v.w[1]), "+v"(v.w[2]), "+v"(v.w[3]));
}

// Element e of a vector, widened to float.
template <typename T>
__device__ __forceinline__ float elem(const Vec &v, int e);

template <>
__device__ __forceinline__ float elem<float>(const Vec &v, int e) {
  return __builtin_bit_cast(float, v.w[e]);
}

template <>
__device__ __forceinline__ float elem<bf16>(const Vec &v, int e) {
  const uint32_t w = v.w[e >> 1];
  // A bfloat16 is the high half of a float32.
  return __builtin_bit_cast(float, (e & 1) ? (w & 0xffff0000u) : (w << 16));
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Pack float values into a storage vector (bfloat16: round to nearest even,
// one v_cvt_pk_bf16_f32 per pair).
template <typename T>
__device__ __forceinline__ Vec pack(const float (&f)[Elems<T>::value]);

template <>
__device__ __forceinline__ Vec pack<float>(const float (&f)[4]) {
  Vec v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v.w[i] = __builtin_bit_cast(uint32_t, f[i]);
  return v;
}

template <>
__device__ __forceinline__ Vec pack<bf16>(const float (&f)[8]) {
  Vec v;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x2 p = {f[2 * i], f[2 * i + 1]};
    v.w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
  }
  return v;
}

// ---------------------------------------------------------------- reductions
//
// Sum across the 64 lanes of a wavefront.  Inside each row of 16 lanes a
// butterfly of four DPP adds (quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror) leaves every lane with its row's sum; the four
// row sums are then read into scalar registers and added in a fixed order.
// Every lane returns the same, wave-uniform value, and the order of the
// additions is fixed, so results are reproducible bit for bit.

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  const int moved = __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false);
  return v + __builtin_bit_cast(float, moved);
}

__device__ __forceinline__ float row16_sum(float v) {
  v = dpp_add<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_add<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_add<0x141>(v);  // row_half_mirror
  v = dpp_add<0x140>(v);  // row_mirror
  return v;
}

__device__ __forceinline__ float lane_read(float v, int lane) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (lane_read(v, 0) + lane_read(v, 16)) +
         (lane_read(v, 32) + lane_read(v, 48));
}

// Two independent sums, interleaved so their DPP chains overlap.
__device__ __forceinline__ void wave_sum2(float &a, float &b) {
  a = dpp_add<0xB1>(a);
  b = dpp_add<0xB1>(b);
  a = dpp_add<0x4E>(a);
  b = dpp_add<0x4E>(b);
  a = dpp_add<0x141>(a);
  b = dpp_add<0x141>(b);
  a = dpp_add<0x140>(a);
  b = dpp_add<0x140>(b);
  a = (lane_read(a, 0) + lane_read(a, 16)) + (lane_read(a, 32) + lane_read(a, 48));
  b = (lane_read(b, 0) + lane_read(b, 16)) + (lane_read(b, 32) + lane_read(b, 48));
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Wave index inside the workgroup, known uniform to the compiler.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

}  // namespace adaln
