// Reductions inside a group of G lanes of one wavefront, shared by the
// routing kernels (gfx950 only).
#pragma once

#include "device_common.h"

namespace moe {

// Butterfly reductions inside a group of G lanes (a power of two, at most
// 64, groups aligned to G lanes).  Steps within a 16-lane row use DPP lane
// moves (quad permutes, then the half-row and row mirrors: after the quad
// steps every lane of a quad holds the same value, so pairing quad q with
// its mirror image combines distinct quads); wider steps use a permute.
// Every lane of the group ends with the same bits (the combining operations
// are commutative).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
template <int G, typename F>
__device__ __forceinline__ uint32_t group_reduce(uint32_t v, F op) {
  if constexpr (G >= 2) v = op(v, dpp<0xB1>(v));    // quad_perm 1,0,3,2
  if constexpr (G >= 4) v = op(v, dpp<0x4E>(v));    // quad_perm 2,3,0,1
  if constexpr (G >= 8) v = op(v, dpp<0x141>(v));   // row_half_mirror
  if constexpr (G >= 16) v = op(v, dpp<0x140>(v));  // row_mirror
  if constexpr (G >= 32) v = op(v, (uint32_t)__shfl_xor((int)v, 16, 64));
  if constexpr (G >= 64) v = op(v, (uint32_t)__shfl_xor((int)v, 32, 64));
  return v;
}
template <int G>
__device__ __forceinline__ float group_max(float v) {
  return __uint_as_float(group_reduce<G>(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  return __uint_as_float(group_reduce<G>(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}
template <int G>
__device__ __forceinline__ int group_or(int v) {
  return (int)group_reduce<G>((uint32_t)v, [](uint32_t a, uint32_t b) { return a | b; });
}
template <int G>
__device__ __forceinline__ int group_and(int v) {
  return (int)group_reduce<G>((uint32_t)v, [](uint32_t a, uint32_t b) { return a & b; });
}
template <int G>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v) {
  auto mx = [](uint64_t a, uint64_t b) { return a > b ? a : b; };
  auto pair = [](uint32_t lo, uint32_t hi) { return ((uint64_t)hi << 32) | lo; };
  if constexpr (G >= 2) v = mx(v, pair(dpp<0xB1>((uint32_t)v), dpp<0xB1>((uint32_t)(v >> 32))));
  if constexpr (G >= 4) v = mx(v, pair(dpp<0x4E>((uint32_t)v), dpp<0x4E>((uint32_t)(v >> 32))));
  if constexpr (G >= 8) v = mx(v, pair(dpp<0x141>((uint32_t)v), dpp<0x141>((uint32_t)(v >> 32))));
  if constexpr (G >= 16) v = mx(v, pair(dpp<0x140>((uint32_t)v), dpp<0x140>((uint32_t)(v >> 32))));
#pragma unroll
  for (int o = 16; o < G; o <<= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, o, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, 64);
    v = mx(v, pair(lo, hi));
  }
  return v;
}

// Ranking key of (value v, expert e): the order-preserving bits of v above
// the complemented id, so a larger key is a larger value, then a smaller id.
// A real key is never 0 (the ordered bits of any non-NaN float, -inf
// included, are nonzero), so 0 can mark an expert that must not be chosen.
__device__ __forceinline__ uint64_t make_key(float v, uint32_t e) {
  return ((uint64_t)ordered_bits(v) << 32) | (uint64_t)(0xffffffffu - e);
}

}  // namespace moe
