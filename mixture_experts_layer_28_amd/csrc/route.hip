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
// Layout: a group of G lanes (a power of two, G * PL >= E with PL = 8, or 16
// for E > 512; G = 1 for E <= 8) owns one row; lane l of the group holds the
// PL consecutive experts l*PL .. l*PL+PL-1 in registers, read with 16-byte
// loads where the row layout allows.  Reductions are butterfly shuffles
// inside the group, so every lane ends with the same bits.  Top-k takes k
// rounds; round j finds the largest (logit, -id) key strictly below the key
// chosen in round j-1, so no per-expert "taken" flags are needed.  Slot j's
// id and probability are kept by lane j % G, which writes them at the end.
//
// Rows with E > 1024 use a one-wave-per-row variant that re-reads the row
// from memory each round instead of caching it.

#include "device_common.h"
#include "group_reduce.h"
#include "launch.h"

namespace moe {
namespace {

// Register-cached path: E <= G * PL <= 1024.  VEC: every lane's PL values
// are one or more aligned 16-byte vectors of the row.  One row (< T) per
// group of G lanes; returning ends this row only.
template <int LDT, int G, int PL, bool VEC>
__device__ __forceinline__ void route_row(
    const typename Storage<LDT>::T* __restrict__ logits, int64_t row, int E,
    int k, int renorm, uint32_t* __restrict__ idx,
    typename Storage<LDT>::T* __restrict__ w, uint32_t* keep = nullptr) {
  using S = typename Storage<LDT>::T;
  const int lane = threadIdx.x % G;
  const S* src = logits + row * (int64_t)E + lane * PL;
  const int e0 = lane * PL;

  float v[PL];
  if constexpr (VEC) {
    constexpr int NE = 16 / sizeof(S);  // elements per 16-byte vector
    static_assert(PL % NE == 0, "whole vectors per lane");
#pragma unroll
    for (int q = 0; q < PL / NE; ++q) {
      S tmp[NE];
      *(u32x4*)tmp = *(const u32x4*)(src + q * NE);
#pragma unroll
      for (int i = 0; i < NE; ++i) v[q * NE + i] = to_f32<LDT>(tmp[i]);
    }
  } else {
#pragma unroll
    for (int m = 0; m < PL; ++m)
      v[m] = e0 + m < E ? to_f32<LDT>(src[m]) : -INFINITY;
  }
  int bad = 0, all_ninf = 1;
#pragma unroll
  for (int m = 0; m < PL; ++m) {
    if (e0 + m < E) {
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
      if (keep) keep[j] = (uint32_t)j;
      w_row[j] = from_f32<LDT>(__builtin_nanf(""));
    }
    return;
  }

  float mx = -INFINITY;
#pragma unroll
  for (int m = 0; m < PL; ++m)
    if (e0 + m < E) mx = fmaxf(mx, v[m]);
  mx = group_max<G>(mx);
  float s = 0.0f;
#pragma unroll
  for (int m = 0; m < PL; ++m)
    if (e0 + m < E) s += expf(v[m] - mx);
  s = group_sum<G>(s);

  // ranking keys, computed once; padding slots get key 0 (never chosen:
  // a real key has ordered bits >= 1 or a nonzero id part)
  uint64_t key[PL];
#pragma unroll
  for (int m = 0; m < PL; ++m)
    key[m] = e0 + m < E ? make_key(v[m], (uint32_t)(e0 + m)) : 0ull;

  // k rounds pick the keys; lane j % G keeps slot j's key and, after the
  // rounds, turns it into an id and a probability (one exp per slot).
  uint64_t kj[PL];
#pragma unroll
  for (int m = 0; m < PL; ++m) kj[m] = 0ull;
  uint64_t prev = ~0ull;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int m = 0; m < PL; ++m)
      if (key[m] < prev && key[m] > best) best = key[m];
    best = group_max_u64<G>(best);
    prev = best;
    if (lane == (j % G)) {
#pragma unroll
      for (int m = 0; m < PL; ++m)
        if (m == j / G) kj[m] = best;
    }
  }
  float pj[PL];
  float part = 0.0f;  // this lane's slots, in slot order
#pragma unroll
  for (int m = 0; m < PL; ++m) {
    pj[m] = 0.0f;
    if (lane + G * m < k) {
      const float vb = from_ordered_bits((uint32_t)(kj[m] >> 32));
      pj[m] = expf(vb - mx) / s;
      part += pj[m];
    }
  }
  const float den = renorm ? group_sum<G>(part) : 1.0f;
#pragma unroll
  for (int m = 0; m < PL; ++m) {
    const int j = lane + G * m;
    if (j < k) {
      idx_row[j] = 0xffffffffu - (uint32_t)kj[m];
      if (keep) keep[j] = 0xffffffffu - (uint32_t)kj[m];
      w_row[j] = from_f32<LDT>(renorm ? pj[m] / den : pj[m]);
    }
  }
}

// Rows are walked in a grid-stride loop over a grid of at most kMaxBlocks
// workgroups, so a launch stays within the 2^32 work-item limit whatever T
// is (a group's rows are uniform across its lanes).
constexpr int64_t kMaxBlocks = 65536;

template <int LDT, int G, int PL, bool VEC>
__global__ __launch_bounds__(256) void route_kernel(
    const typename Storage<LDT>::T* __restrict__ logits, int64_t T, int E,
    int k, int renorm, uint32_t* __restrict__ idx,
    typename Storage<LDT>::T* __restrict__ w) {
  constexpr int R = 256 / G;
  for (int64_t row = (int64_t)blockIdx.x * R + threadIdx.x / G; row < T;
       row += (int64_t)gridDim.x * R)
    route_row<LDT, G, PL, VEC>(logits, row, E, k, renorm, idx, w);
}

// Routing and the dispatch count in one launch (the forward's first two
// kernels): workgroup b takes chunk c = b, b + grid, ... of the dispatch
// plan, whose `chunk` entries are chunk / k whole tokens (k divides the
// chunk).  Its groups route those tokens as route_kernel does, also keeping
// the expert ids in LDS; then wavefront 0 counts the chunk exactly as
// dispatch_count_kernel counts it (same table row, same ranks), reading the
// ids from LDS.  LDS: chunk ids + E + 1 counters.
template <int LDT, int G, int PL, bool VEC>
__global__ __launch_bounds__(256) void route_count_kernel(
    const typename Storage<LDT>::T* __restrict__ logits, int64_t T, int E,
    int k, int renorm, uint32_t* __restrict__ idx,
    typename Storage<LDT>::T* __restrict__ w, int64_t chunk, int64_t nchunks,
    uint32_t* __restrict__ table, uint32_t* __restrict__ local_rank) {
  extern __shared__ uint32_t sm[];
  uint32_t* ids = sm;
  uint32_t* cnt = sm + chunk;
  constexpr int R = 256 / G;  // rows per pass of the workgroup
  const int64_t tpc = chunk / k;
  const int64_t N = T * (int64_t)k;
  const int nb = E + 1;
  const int lane = threadIdx.x % 64;
  for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
    const int64_t tok0 = c * tpc;
    for (int64_t r = threadIdx.x / G; r < tpc; r += R) {
      if (tok0 + r < T)  // uniform across the row's group
        route_row<LDT, G, PL, VEC>(logits, tok0 + r, E, k, renorm, idx, w,
                                   ids + r * k);
    }
    __syncthreads();  // the chunk's ids are in LDS
    if (threadIdx.x < 64) {
      for (int b = lane; b < nb; b += 64) cnt[b] = 0u;
      const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
      const int nbits = 32 - __builtin_clz((unsigned)E | 1u);
      const int64_t i0 = c * chunk;
      const int64_t i1 = (i0 + chunk < N) ? i0 + chunk : N;
      for (int64_t g = i0; g < i1; g += 64) {
        const int64_t i = g + lane;
        const bool valid = i < i1;
        uint32_t e = valid ? ids[i - i0] : 0u;
        if (e > (uint32_t)E) e = (uint32_t)E;
        uint64_t same = __ballot(valid);
        for (int bit = 0; bit < nbits; ++bit) {
          const uint64_t m = __ballot(valid && ((e >> bit) & 1u));
          same &= ((e >> bit) & 1u) ? m : ~m;
        }
        const int leader = valid ? (int)__builtin_ctzll(same) : lane;
        uint32_t old = 0;
        if (valid && leader == lane) {
          old = cnt[e];
          cnt[e] = old + (uint32_t)__popcll(same);
        }
        old = (uint32_t)__shfl((int)old, leader, 64);
        if (valid) local_rank[i] = old + (uint32_t)__popcll(same & lt);
      }
      for (int b = lane; b < nb; b += 64) table[c * nb + b] = cnt[b];
    }
    __syncthreads();  // LDS free for the next chunk
  }
}

// Wide rows (E > 1024): one wave per row, values re-read each round; with
// renormalisation a first pass over the k rounds computes the denominator.
template <int LDT>
__device__ __forceinline__ void route_wide_row(
    const typename Storage<LDT>::T* __restrict__ logits, int64_t row, int E,
    int k, int renorm, uint32_t* __restrict__ idx,
    typename Storage<LDT>::T* __restrict__ w) {
  using S = typename Storage<LDT>::T;
  constexpr int G = 64;
  const int lane = threadIdx.x % G;
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

template <int LDT>
__global__ __launch_bounds__(256) void route_wide_kernel(
    const typename Storage<LDT>::T* __restrict__ logits, int64_t T, int E,
    int k, int renorm, uint32_t* __restrict__ idx,
    typename Storage<LDT>::T* __restrict__ w) {
  for (int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / 64; row < T;
       row += (int64_t)gridDim.x * 4)
    route_wide_row<LDT>(logits, row, E, k, renorm, idx, w);
}

template <int LDT, int G, int PL>
hipError_t launch_g(const void* logits, int64_t T, int E, int k, int renorm,
                    uint32_t* idx, void* w, hipStream_t st) {
  using S = typename Storage<LDT>::T;
  const int rows = 256 / G;
  const int64_t blocks = (T + rows - 1) / rows;
  const dim3 grid((unsigned)(blocks < kMaxBlocks ? blocks : kMaxBlocks));
  // 16-byte loads when every lane's PL values are whole aligned vectors
  const bool vec = (PL * sizeof(S)) % 16 == 0 && E == G * PL &&
                   (uintptr_t)logits % 16 == 0;
  if (vec)
    hipLaunchKernelGGL((route_kernel<LDT, G, PL, true>), grid, dim3(256), 0,
                       st, (const S*)logits, T, E, k, renorm, idx, (S*)w);
  else
    hipLaunchKernelGGL((route_kernel<LDT, G, PL, false>), grid, dim3(256), 0,
                       st, (const S*)logits, T, E, k, renorm, idx, (S*)w);
  return hipGetLastError();
}

template <int LDT>
hipError_t launch_route_t(const void* logits, int64_t T, int E, int k,
                          int renorm, uint32_t* idx, void* w, hipStream_t st) {
  using S = typename Storage<LDT>::T;
  if (E <= 8) return launch_g<LDT, 1, 8>(logits, T, E, k, renorm, idx, w, st);
  if (E <= 16) return launch_g<LDT, 2, 8>(logits, T, E, k, renorm, idx, w, st);
  if (E <= 32) return launch_g<LDT, 4, 8>(logits, T, E, k, renorm, idx, w, st);
  if (E <= 64) return launch_g<LDT, 8, 8>(logits, T, E, k, renorm, idx, w, st);
  if (E <= 128) return launch_g<LDT, 16, 8>(logits, T, E, k, renorm, idx, w, st);
  if (E <= 256) return launch_g<LDT, 32, 8>(logits, T, E, k, renorm, idx, w, st);
  if (E <= 512) return launch_g<LDT, 64, 8>(logits, T, E, k, renorm, idx, w, st);
  if (E <= 1024) return launch_g<LDT, 64, 16>(logits, T, E, k, renorm, idx, w, st);
  const int64_t blocks = (T + 3) / 4;
  const dim3 grid((unsigned)(blocks < kMaxBlocks ? blocks : kMaxBlocks));
  hipLaunchKernelGGL((route_wide_kernel<LDT>), grid, dim3(256), 0, st,
                     (const S*)logits, T, E, k, renorm, idx, (S*)w);
  return hipGetLastError();
}

template <int LDT, int G, int PL>
hipError_t launch_gc(const void* logits, int64_t T, int E, int k, int renorm,
                     uint32_t* idx, void* w, const DispatchPlan& p,
                     uint32_t* table, uint32_t* local_rank, hipStream_t st) {
  using S = typename Storage<LDT>::T;
  const dim3 grid((unsigned)(p.nchunks < kMaxBlocks ? p.nchunks : kMaxBlocks));
  const size_t lds = (size_t)(p.chunk + E + 1) * sizeof(uint32_t);
  const bool vec = (PL * sizeof(S)) % 16 == 0 && E == G * PL &&
                   (uintptr_t)logits % 16 == 0;
  if (vec)
    hipLaunchKernelGGL((route_count_kernel<LDT, G, PL, true>), grid, dim3(256),
                       lds, st, (const S*)logits, T, E, k, renorm, idx, (S*)w,
                       p.chunk, p.nchunks, table, local_rank);
  else
    hipLaunchKernelGGL((route_count_kernel<LDT, G, PL, false>), grid, dim3(256),
                       lds, st, (const S*)logits, T, E, k, renorm, idx, (S*)w,
                       p.chunk, p.nchunks, table, local_rank);
  return hipGetLastError();
}

template <int LDT>
hipError_t launch_route_count_t(const void* logits, int64_t T, int E, int k,
                                int renorm, uint32_t* idx, void* w,
                                const DispatchPlan& p, uint32_t* table,
                                uint32_t* rank, hipStream_t st) {
#define MOE_RC(G, PL) \
  launch_gc<LDT, G, PL>(logits, T, E, k, renorm, idx, w, p, table, rank, st)
  if (E <= 8) return MOE_RC(1, 8);
  if (E <= 16) return MOE_RC(2, 8);
  if (E <= 32) return MOE_RC(4, 8);
  if (E <= 64) return MOE_RC(8, 8);
  if (E <= 128) return MOE_RC(16, 8);
  if (E <= 256) return MOE_RC(32, 8);
  if (E <= 512) return MOE_RC(64, 8);
  return MOE_RC(64, 16);
#undef MOE_RC
}

}  // namespace

bool route_count_fusable(int E, int k, const DispatchPlan& p) {
  if (E < 1 || E > kMaxFusedE || k < 1 || p.nchunks <= 0 ||
      p.chunk % k != 0 || p.chunk + E + 1 > kMaxFusedLds)
    return false;
  // lanes per row as launch_route_count_t picks them; at most 4 passes of
  // 256 / G rows per chunk (beyond that the separate routing launch, with
  // a workgroup per 256 / G rows, spreads the rows wider)
  int G = 1;
  while (G < 64 && G * 8 < E) G *= 2;
  return p.chunk / k <= 4 * (256 / G);
}

hipError_t launch_route_count(const void* logits, int ldt, int64_t T, int E,
                              int k, int renorm, uint32_t* idx, void* w,
                              const DispatchPlan& p, uint32_t* table,
                              uint32_t* local_rank, hipStream_t st) {
  if (!route_count_fusable(E, k, p)) return hipErrorInvalidValue;
  switch (ldt) {
    case DT_F32: return launch_route_count_t<DT_F32>(logits, T, E, k, renorm, idx, w, p, table, local_rank, st);
    case DT_F16: return launch_route_count_t<DT_F16>(logits, T, E, k, renorm, idx, w, p, table, local_rank, st);
    default: return launch_route_count_t<DT_BF16>(logits, T, E, k, renorm, idx, w, p, table, local_rank, st);
  }
}

hipError_t launch_route(const void* logits, int ldt, int64_t T, int E, int k,
                        int renorm, uint32_t* idx, void* w, hipStream_t st) {
  switch (ldt) {
    case DT_F32: return launch_route_t<DT_F32>(logits, T, E, k, renorm, idx, w, st);
    case DT_F16: return launch_route_t<DT_F16>(logits, T, E, k, renorm, idx, w, st);
    default: return launch_route_t<DT_BF16>(logits, T, E, k, renorm, idx, w, st);
  }
}

}  // namespace moe
