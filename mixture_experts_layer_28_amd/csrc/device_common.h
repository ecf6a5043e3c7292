// Device-side helpers shared by the libmoe kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum Dt { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

// Storage type of each dtype code.  Conversions to storage use the
// hardware converts, which round to nearest even (v_cvt_f16_f32 under the
// default round mode, v_cvt_pk_bf16_f32 on gfx950) and keep NaN a NaN.
template <int D> struct Storage;
template <> struct Storage<DT_F32> { using T = float; };
template <> struct Storage<DT_F16> { using T = _Float16; };
template <> struct Storage<DT_BF16> { using T = __bf16; };

template <int D>
__device__ __forceinline__ float to_f32(typename Storage<D>::T v) {
  return static_cast<float>(v);
}
template <int D>
__device__ __forceinline__ typename Storage<D>::T from_f32(float v) {
  return static_cast<typename Storage<D>::T>(v);
}

// Float -> unsigned key whose unsigned order is the float order (NaN
// excluded by the callers).  -0 is folded onto +0 first so that equal
// values tie exactly.
__device__ __forceinline__ uint32_t ordered_bits(float v) {
  if (v == 0.0f) v = 0.0f;
  uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered_bits(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(u);
}

// Values every lane of a wavefront agrees on (e.g. read back from LDS) held
// in scalar registers: the compiler cannot prove such loads uniform, and a
// buffer descriptor built from a "divergent" value forces a loop over lanes
// around every buffer instruction.
__device__ __forceinline__ int uniform(int v) {
  return __builtin_amdgcn_readfirstlane(v);
}
__device__ __forceinline__ int64_t uniform(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Logical workgroup id that keeps consecutive ids on one XCD.  The
// dispatcher deals workgroups to the 8 XCDs of an MI355X round-robin, so
// hardware id b runs on XCD b % 8; this renumbers so XCD x owns the
// contiguous range of logical ids [start(x), start(x) + count(x)).
__device__ __forceinline__ uint32_t xcd_logical_id(uint32_t b, uint32_t G) {
  const uint32_t q = G / 8u, r = G % 8u, x = b % 8u;
  return x * q + (x < r ? x : r) + b / 8u;
}

}  // namespace moe
