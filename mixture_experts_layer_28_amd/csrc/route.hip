// Routing kernel: FP32 softmax over all experts, then top-k.
//
// Contract: ruDNN user guide (RUDA docs), section 4 "routing contract".
// The softmax runs over all E experts in FP32 before top-k; ties go to the
// lower expert id; selected weights are optionally renormalised and then
// rounded to the logits dtype; a row holding NaN, +inf or only -inf keeps
// NaN weights (its indices are 0..k-1: with no order among NaN
// probabilities every expert ties, and ties go to lower ids).
//
// Ranking key: the FP32 logit, descending, then the id, ascending.  The
// softmax is strictly increasing in the logit, so this is the exact order of
// the softmax values, and it is decided on exact data (no exp rounding).
//
// Layout: a group of G lanes (G = 8..64, a power of two >= min(E, 64))
// owns one row; lane l of the group holds experts l, l+G, l+2G, ... in
// registers.  Reductions are butterfly shuffles inside the group, so every
// lane ends with the same bits.  Top-k takes k rounds; round j finds the
// largest (logit, -id) key strictly below the key chosen in round j-1, so no
// per-expert "taken" flags are needed.  Slot j's id and probability are kept
// by lane j % G, which writes them at the end (coalesced).
//
// Rows with E > 1024 use a one-wave-per-row variant that re-reads the row
// from memory each round instead of caching it.

#include "device_common.h"
#include "launch.h"

namespace moe {
namespace {

template <int G>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, G));
  return v;
}
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, G);
  return v;
}
template <int G>
__device__ __forceinline__ int group_or(int v) {
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) v |= __shfl_xor(v, o, G);
  return v;
}
template <int G>
__device__ __forceinline__ int group_and(int v) {
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) v &= __shfl_xor(v, o, G);
  return v;
}
template <int G>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v) {
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, o, G);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, G);
    uint64_t w = ((uint64_t)hi << 32) | lo;
    v = w > v ? w : v;
  }
  return v;
}

__device__ __forceinline__ uint64_t make_key(float v, uint32_t e) {
  return ((uint64_t)ordered_bits(v) << 32) | (uint64_t)(0xffffffffu - e);
}

// Register-cached path: E <= G * PL <= 1024.
template <int LDT, int G, int PL>
__global__ __launch_bounds__(256) void route_kernel(
    const typename Storage<LDT>::T* __restrict__ logits, int64_t T, int E,
    int k, int renorm, uint32_t* __restrict__ idx,
    typename Storage<LDT>::T* __restrict__ w) {
  using S = typename Storage<LDT>::T;
  const int lane = threadIdx.x % G;
  const int64_t row = (int64_t)blockIdx.x * (256 / G) + threadIdx.x / G;
  if (row >= T) return;  // uniform across the group
  const S* src = logits + row * (int64_t)E;

  float v[PL];
  int bad = 0, all_ninf = 1;
#pragma unroll
  for (int m = 0; m < PL; ++m) {
    const int e = lane + G * m;
    v[m] = -INFINITY;
    if (e < E) {
      v[m] = to_f32<LDT>(src[e]);
      bad |= (__builtin_isnan(v[m]) || v[m] == INFINITY);
      all_ninf &= (v[m] == -INFINITY);
    }
  }
  bad = group_or<G>(bad) | group_and<G>(all_ninf);

  uint32_t* idx_row = idx + row * (int64_t)k;
  S* w_row = w + row * (int64_t)k;
  if (bad) {
    for (int j = lane; j < k; j += G) {
      idx_row[j] = (uint32_t)j;
      w_row[j] = from_f32<LDT>(__builtin_nanf(""));
    }
    return;
  }

  float mx = -INFINITY;
#pragma unroll
  for (int m = 0; m < PL; ++m)
    if (lane + G * m < E) mx = fmaxf(mx, v[m]);
  mx = group_max<G>(mx);
  float s = 0.0f;
#pragma unroll
  for (int m = 0; m < PL; ++m)
    if (lane + G * m < E) s += expf(v[m] - mx);
  s = group_sum<G>(s);

  float pj[PL];
  uint32_t ej[PL];
#pragma unroll
  for (int m = 0; m < PL; ++m) { pj[m] = 0.0f; ej[m] = 0u; }
  uint64_t prev = ~0ull;
  float den = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int m = 0; m < PL; ++m) {
      const int e = lane + G * m;
      if (e < E) {
        const uint64_t key = make_key(v[m], (uint32_t)e);
        if (key < prev && key > best) best = key;
      }
    }
    best = group_max_u64<G>(best);
    prev = best;
    const uint32_t eb = 0xffffffffu - (uint32_t)best;
    const float vb = from_ordered_bits((uint32_t)(best >> 32));
    const float p = expf(vb - mx) / s;
    den += p;  // slot order, identical on every lane
    if (lane == (j % G)) {
#pragma unroll
      for (int m = 0; m < PL; ++m)
        if (m == j / G) { pj[m] = p; ej[m] = eb; }
    }
  }
#pragma unroll
  for (int m = 0; m < PL; ++m) {
    const int j = lane + G * m;
    if (j < k) {
      idx_row[j] = ej[m];
      w_row[j] = from_f32<LDT>(renorm ? pj[m] / den : pj[m]);
    }
  }
}

// Wide rows (E > 1024): one wave per row, values re-read each round; with
// renormalisation a first pass over the k rounds computes the denominator.
template <int LDT>
__global__ __launch_bounds__(256) void route_wide_kernel(
    const typename Storage<LDT>::T* __restrict__ logits, int64_t T, int E,
    int k, int renorm, uint32_t* __restrict__ idx,
    typename Storage<LDT>::T* __restrict__ w) {
  using S = typename Storage<LDT>::T;
  constexpr int G = 64;
  const int lane = threadIdx.x % G;
  const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / G;
  if (row >= T) return;
  const S* src = logits + row * (int64_t)E;
  uint32_t* idx_row = idx + row * (int64_t)k;
  S* w_row = w + row * (int64_t)k;

  int bad = 0, all_ninf = 1;
  float mx = -INFINITY;
  for (int e = lane; e < E; e += G) {
    const float x = to_f32<LDT>(src[e]);
    bad |= (__builtin_isnan(x) || x == INFINITY);
    all_ninf &= (x == -INFINITY);
    mx = fmaxf(mx, x);
  }
  bad = group_or<G>(bad) | group_and<G>(all_ninf);
  if (bad) {
    for (int j = lane; j < k; j += G) {
      idx_row[j] = (uint32_t)j;
      w_row[j] = from_f32<LDT>(__builtin_nanf(""));
    }
    return;
  }
  mx = group_max<G>(mx);
  float s = 0.0f;
  for (int e = lane; e < E; e += G) s += expf(to_f32<LDT>(src[e]) - mx);
  s = group_sum<G>(s);

  float den = 1.0f;
  for (int pass = renorm ? 0 : 1; pass < 2; ++pass) {
    uint64_t prev = ~0ull;
    float acc = 0.0f;
    for (int j = 0; j < k; ++j) {
      uint64_t best = 0;
      for (int e = lane; e < E; e += G) {
        const uint64_t key = make_key(to_f32<LDT>(src[e]), (uint32_t)e);
        if (key < prev && key > best) best = key;
      }
      best = group_max_u64<G>(best);
      prev = best;
      const float vb = from_ordered_bits((uint32_t)(best >> 32));
      const float p = expf(vb - mx) / s;
      if (pass == 0) {
        acc += p;
      } else if (lane == 0) {
        idx_row[j] = 0xffffffffu - (uint32_t)best;
        w_row[j] = from_f32<LDT>(renorm ? p / den : p);
      }
    }
    if (pass == 0) den = acc;
  }
}

template <int LDT, int G, int PL>
hipError_t launch_g(const void* logits, int64_t T, int E, int k, int renorm,
                    uint32_t* idx, void* w, hipStream_t st) {
  using S = typename Storage<LDT>::T;
  const int rows = 256 / G;
  const dim3 grid((unsigned)((T + rows - 1) / rows));
  hipLaunchKernelGGL((route_kernel<LDT, G, PL>), grid, dim3(256), 0, st,
                     (const S*)logits, T, E, k, renorm, idx, (S*)w);
  return hipGetLastError();
}

template <int LDT>
hipError_t launch_route_t(const void* logits, int64_t T, int E, int k,
                          int renorm, uint32_t* idx, void* w, hipStream_t st) {
  using S = typename Storage<LDT>::T;
  if (E <= 8) return launch_g<LDT, 8, 1>(logits, T, E, k, renorm, idx, w, st);
  if (E <= 16) return launch_g<LDT, 16, 1>(logits, T, E, k, renorm, idx, w, st);
  if (E <= 32) return launch_g<LDT, 32, 1>(logits, T, E, k, renorm, idx, w, st);
  if (E <= 64) return launch_g<LDT, 64, 1>(logits, T, E, k, renorm, idx, w, st);
  if (E <= 128) return launch_g<LDT, 64, 2>(logits, T, E, k, renorm, idx, w, st);
  if (E <= 256) return launch_g<LDT, 64, 4>(logits, T, E, k, renorm, idx, w, st);
  if (E <= 512) return launch_g<LDT, 64, 8>(logits, T, E, k, renorm, idx, w, st);
  if (E <= 1024) return launch_g<LDT, 64, 16>(logits, T, E, k, renorm, idx, w, st);
  const dim3 grid((unsigned)((T + 3) / 4));
  hipLaunchKernelGGL((route_wide_kernel<LDT>), grid, dim3(256), 0, st,
                     (const S*)logits, T, E, k, renorm, idx, (S*)w);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const void* logits, int ldt, int64_t T, int E, int k,
                        int renorm, uint32_t* idx, void* w, hipStream_t st) {
  switch (ldt) {
    case DT_F32: return launch_route_t<DT_F32>(logits, T, E, k, renorm, idx, w, st);
    case DT_F16: return launch_route_t<DT_F16>(logits, T, E, k, renorm, idx, w, st);
    default: return launch_route_t<DT_BF16>(logits, T, E, k, renorm, idx, w, st);
  }
}

}  // namespace moe
