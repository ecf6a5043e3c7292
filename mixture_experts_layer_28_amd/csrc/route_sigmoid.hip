// Group-limited sigmoid routing.
//
// Contract: ruDNN user guide (RUDA docs, German edition), section 10
// "group-limited sigmoid MoE routing" (route_sigmoid_grouped with
// GroupRoutingOptions).  Scores are FP32 sigmoids of the logits; an
// optional FP32 correction bias is added for the selection only; the
// experts form `groups` equal groups of consecutive ids, each scored by its
// largest corrected value or, with group_top_two, by the sum of its two
// largest; the `selected_groups` best groups are kept and top_k experts are
// chosen among them; the weights are the uncorrected sigmoid values,
// optionally renormalised over the chosen experts, times `scale`, rounded to
// the logits dtype.  Ties (experts and groups) go to the smaller id.  A row
// whose corrected values or group scores hold a NaN has no order: its
// indices are 0..k-1 and its weights NaN.
//
// Precision: the sigmoid is evaluated in float64 and rounded once to
// float32, which gives the correctly rounded FP32 sigmoid except when the
// float64 value lies within a few float64 ulps of a float32 rounding
// boundary (~1e-9 of values).  The selection compares these values, so it
// agrees with any other correctly rounded evaluation.  The renormalising
// sum runs over the chosen experts in slot order.
//
// Layout: G lanes own a row (G * PL >= E, the same split as the softmax
// router); lane l computes the scores of experts l*PL .. l*PL+PL-1 and keeps
// the corrected values in registers for the top-k rounds.  The group stage
// goes through LDS, so any group size works: each group is split over
// P = max(1, G / groups) lanes that scan a strided share of its corrected
// values for the two largest, then one lane per group merges the P partial
// pairs into the group score.  A group is kept iff fewer than
// selected_groups groups beat it (counted over the row's group scores).
// Top-k then takes k rounds of a 64-bit key maximum over the kept experts,
// as in the softmax router; chosen ids go to LDS so that every lane can form
// the slot-ordered renormalising sum.  When the groups are whole lanes
// (route_sigmoid_lane_kernel) the group stage runs in registers instead.
//
// Rows are walked in a grid-stride loop, so the grid stays a fixed size
// whatever T is, and every barrier is reached by all threads of a block.

#include "device_common.h"
#include "group_reduce.h"
#include "launch.h"

namespace moe {
namespace {

__device__ __forceinline__ float sigmoid_f32(float x) {
#pragma clang fp contract(off)
  const double e = exp(-(double)x);
  return (float)(1.0 / (1.0 + e));
}

template <int LDT, int G, int PL, bool VEC>
__global__ __launch_bounds__(256) void route_sigmoid_kernel(
    const typename Storage<LDT>::T* __restrict__ logits,
    const float* __restrict__ bias, int64_t T, int E, int k,
    GroupRouting o, uint32_t* __restrict__ idx,
    typename Storage<LDT>::T* __restrict__ w) {
  using S = typename Storage<LDT>::T;
  constexpr int R = 256 / G;   // rows per block and pass
  constexpr int W = G * PL;    // LDS words per row (>= E)
  __shared__ float cl[R * W];  // corrected values
  __shared__ float sl[R * W];  // sigmoid values
  __shared__ float p1[R * W];  // partial largest values, then kept flags
  __shared__ float p2[R * W];  // partial second-largest values
  __shared__ float gl[R * W];  // group scores, then chosen ids
  int* kept = (int*)p1;
  uint32_t* chosen = (uint32_t*)gl;

  const int lane = threadIdx.x % G;
  const int rb = (int)(threadIdx.x / G) * W;
  const int e0 = lane * PL;
  const int P = o.groups >= G ? 1 : G / o.groups;
  const int ntask = o.groups * P;  // <= max(groups, G) <= W

  for (int64_t base = (int64_t)blockIdx.x * R; base < T;
       base += (int64_t)gridDim.x * R) {
    const int64_t row = base + threadIdx.x / G;
    const bool live = row < T;

    // scores
    float v[PL];
    if (live) {
      const S* src = logits + row * (int64_t)E + e0;
      if constexpr (VEC) {
        constexpr int NE = 16 / sizeof(S);
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
          v[m] = e0 + m < E ? to_f32<LDT>(src[m]) : 0.0f;
      }
    } else {
#pragma unroll
      for (int m = 0; m < PL; ++m) v[m] = 0.0f;
    }
    float c[PL];
    int bad = 0;
#pragma unroll
    for (int m = 0; m < PL; ++m) {
      const int e = e0 + m;
      c[m] = -INFINITY;
      if (e < E) {
        const float s = sigmoid_f32(v[m]);
        c[m] = bias ? s + bias[e] : s;
        bad |= __builtin_isnan(c[m]);
        sl[rb + e] = s;
        cl[rb + e] = c[m];
      }
    }
    __syncthreads();

    // group scores: partial top-two over a strided share of each group
    for (int t = lane; t < ntask; t += G) {
      const float* cg = cl + rb + (t / P) * o.gsz;
      float a = -INFINITY, b = -INFINITY;
      for (int j = t % P; j < o.gsz; j += P) {
        const float x = cg[j];
        if (x > a) {
          b = a;
          a = x;
        } else if (x > b) {
          b = x;
        }
      }
      p1[rb + t] = a;
      p2[rb + t] = b;
    }
    __syncthreads();
    for (int g = lane; g < o.groups; g += G) {
      float a = -INFINITY, b = -INFINITY;  // a >= b; merge pairs (x1 >= x2)
      for (int p = 0; p < P; ++p) {
        const float x1 = p1[rb + g * P + p], x2 = p2[rb + g * P + p];
        if (x1 > a) {
          b = fmaxf(a, x2);
          a = x1;
        } else {
          b = fmaxf(b, x1);
        }
      }
      gl[rb + g] = o.top_two ? a + b : a;
    }
    __syncthreads();

    // kept groups: fewer than selected_groups groups rank before this one
    for (int g = lane; g < o.groups; g += G) {
      const float x = gl[rb + g];
      bad |= __builtin_isnan(x);
      int beat = 0;
      for (int h = 0; h < o.groups; ++h) {
        const float y = gl[rb + h];
        beat += (y > x) || (y == x && h < g);
      }
      kept[rb + g] = beat < o.selected;
    }
    bad = group_or<G>(bad);
    __syncthreads();

    // top-k among the kept experts; lane j % G keeps slot j's key
    uint64_t kj[PL];
#pragma unroll
    for (int m = 0; m < PL; ++m) kj[m] = 0ull;
    if (live && !bad) {
      uint64_t key[PL];
#pragma unroll
      for (int m = 0; m < PL; ++m) {
        const int e = e0 + m;
        key[m] = e < E && kept[rb + e / o.gsz]
                     ? make_key(c[m], (uint32_t)e) : 0ull;
      }
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
#pragma unroll
      for (int m = 0; m < PL; ++m)
        if (lane + G * m < k)
          chosen[rb + lane + G * m] = 0xffffffffu - (uint32_t)kj[m];
    }
    __syncthreads();

    if (live) {
      uint32_t* idx_row = idx + row * (int64_t)k;
      S* w_row = w + row * (int64_t)k;
      if (bad) {
        for (int j = lane; j < k; j += G) {
          idx_row[j] = (uint32_t)j;
          w_row[j] = from_f32<LDT>(__builtin_nanf(""));
        }
      } else {
        float den = 1.0f;
        if (o.renorm) {
          den = 0.0f;
          for (int j = 0; j < k; ++j) den += sl[rb + chosen[rb + j]];
        }
#pragma unroll
        for (int m = 0; m < PL; ++m) {
          const int j = lane + G * m;
          if (j < k) {
            const uint32_t e = chosen[rb + j];
            float x = sl[rb + e];
            if (o.renorm) x = x / den;
            idx_row[j] = e;
            w_row[j] = from_f32<LDT>(x * o.scale);
          }
        }
      }
    }
    // the next pass overwrites this pass's LDS rows
    __syncthreads();
  }
}

// Lane-aligned groups: E == G * PL and each group is L = gsz / PL whole
// lanes (L a power of two).  Every step then stays in registers: a lane's
// top two, merged over its group's L lanes by butterfly shuffles; each
// group's rank counted over the other groups' scores fetched by shuffles;
// the k rounds as above; the chosen experts' sigmoid values broadcast slot
// by slot from their owner lanes, so every lane forms the slot-ordered
// renormalising sum.  No LDS and no barriers.
template <int LDT, int G, int PL, bool VEC>
__global__ __launch_bounds__(256) void route_sigmoid_lane_kernel(
    const typename Storage<LDT>::T* __restrict__ logits,
    const float* __restrict__ bias, int64_t T, int E, int k,
    GroupRouting o, int L, uint32_t* __restrict__ idx,
    typename Storage<LDT>::T* __restrict__ w) {
  using S = typename Storage<LDT>::T;
  constexpr int R = 256 / G;
  const int lane = threadIdx.x % G;
  const int first = (int)(threadIdx.x % 64) - lane;  // the row's first lane
  const int e0 = lane * PL;
  const int g = lane / L;  // this lane's group

  for (int64_t row = (int64_t)blockIdx.x * R + threadIdx.x / G; row < T;
       row += (int64_t)gridDim.x * R) {
    const S* src = logits + row * (int64_t)E + e0;
    float v[PL];
    if constexpr (VEC) {
      constexpr int NE = 16 / sizeof(S);
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
      for (int m = 0; m < PL; ++m) v[m] = to_f32<LDT>(src[m]);
    }
    float sg[PL], c[PL];
    int bad = 0;
    float a = -INFINITY, b = -INFINITY;  // this lane's two largest c
#pragma unroll
    for (int m = 0; m < PL; ++m) {
      sg[m] = sigmoid_f32(v[m]);
      c[m] = bias ? sg[m] + bias[e0 + m] : sg[m];
      bad |= __builtin_isnan(c[m]);
      if (c[m] > a) {
        b = a;
        a = c[m];
      } else if (c[m] > b) {
        b = c[m];
      }
    }
    // the group's two largest: merge the pairs of its L lanes
    for (int off = 1; off < L; off <<= 1) {
      const float a2 = __shfl_xor(a, off, 64), b2 = __shfl_xor(b, off, 64);
      if (a2 > a) {
        b = fmaxf(a, b2);
        a = a2;
      } else {
        b = fmaxf(b, a2);
      }
    }
    const float score = o.top_two ? a + b : a;
    bad |= __builtin_isnan(score);
    int beat = 0;
    for (int h = 0; h < o.groups; ++h) {
      const float y = __shfl(score, first + h * L, 64);
      beat += (y > score) || (y == score && h < g);
    }
    const bool kept = beat < o.selected;
    bad = group_or<G>(bad);

    uint32_t* idx_row = idx + row * (int64_t)k;
    S* w_row = w + row * (int64_t)k;
    if (bad) {
      for (int j = lane; j < k; j += G) {
        idx_row[j] = (uint32_t)j;
        w_row[j] = from_f32<LDT>(__builtin_nanf(""));
      }
      continue;
    }
    uint64_t key[PL];
#pragma unroll
    for (int m = 0; m < PL; ++m)
      key[m] = kept ? make_key(c[m], (uint32_t)(e0 + m)) : 0ull;
    uint64_t kj[PL];
#pragma unroll
    for (int m = 0; m < PL; ++m) kj[m] = 0ull;
    uint64_t prev = ~0ull;
    float den = 0.0f;
    float sv[PL];
#pragma unroll
    for (int m = 0; m < PL; ++m) sv[m] = 0.0f;
    for (int j = 0; j < k; ++j) {
      uint64_t best = 0;
#pragma unroll
      for (int m = 0; m < PL; ++m)
        if (key[m] < prev && key[m] > best) best = key[m];
      best = group_max_u64<G>(best);
      prev = best;
      // the chosen expert's sigmoid value, from the lane that holds it
      const uint32_t id = 0xffffffffu - (uint32_t)best;
      const int m_id = (int)(id % PL);
      float mine = 0.0f;
#pragma unroll
      for (int m = 0; m < PL; ++m)
        if (m == m_id) mine = sg[m];
      const float sj = __shfl(mine, first + (int)(id / PL), 64);
      den += sj;
      if (lane == (j % G)) {
#pragma unroll
        for (int m = 0; m < PL; ++m)
          if (m == j / G) {
            kj[m] = best;
            sv[m] = sj;
          }
      }
    }
#pragma unroll
    for (int m = 0; m < PL; ++m) {
      const int j = lane + G * m;
      if (j < k) {
        float x = sv[m];
        if (o.renorm) x = x / den;
        idx_row[j] = 0xffffffffu - (uint32_t)kj[m];
        w_row[j] = from_f32<LDT>(x * o.scale);
      }
    }
  }
}

template <int LDT, int G, int PL>
hipError_t launch_sg(const void* logits, const float* bias, int64_t T, int E,
                     int k, const GroupRouting& o, uint32_t* idx, void* w,
                     hipStream_t st) {
  using S = typename Storage<LDT>::T;
  constexpr int R = 256 / G;
  const int64_t blocks = (T + R - 1) / R;
  const dim3 grid((unsigned)(blocks < 65536 ? blocks : 65536));
  const bool vec = (PL * sizeof(S)) % 16 == 0 && E == G * PL &&
                   (uintptr_t)logits % 16 == 0;
  // lane-aligned groups: whole lanes per group, a power of two of them
  const int L = o.gsz / PL;
  if (E == G * PL && o.gsz % PL == 0 && (L & (L - 1)) == 0) {
    if (vec)
      hipLaunchKernelGGL((route_sigmoid_lane_kernel<LDT, G, PL, true>), grid,
                         dim3(256), 0, st, (const S*)logits, bias, T, E, k, o,
                         L, idx, (S*)w);
    else
      hipLaunchKernelGGL((route_sigmoid_lane_kernel<LDT, G, PL, false>), grid,
                         dim3(256), 0, st, (const S*)logits, bias, T, E, k, o,
                         L, idx, (S*)w);
    return hipGetLastError();
  }
  if (vec)
    hipLaunchKernelGGL((route_sigmoid_kernel<LDT, G, PL, true>), grid,
                       dim3(256), 0, st, (const S*)logits, bias, T, E, k, o,
                       idx, (S*)w);
  else
    hipLaunchKernelGGL((route_sigmoid_kernel<LDT, G, PL, false>), grid,
                       dim3(256), 0, st, (const S*)logits, bias, T, E, k, o,
                       idx, (S*)w);
  return hipGetLastError();
}

template <int LDT>
hipError_t launch_sigmoid_t(const void* logits, const float* bias, int64_t T,
                            int E, int k, const GroupRouting& o,
                            uint32_t* idx, void* w, hipStream_t st) {
  if (E <= 8) return launch_sg<LDT, 1, 8>(logits, bias, T, E, k, o, idx, w, st);
  if (E <= 16) return launch_sg<LDT, 2, 8>(logits, bias, T, E, k, o, idx, w, st);
  if (E <= 32) return launch_sg<LDT, 4, 8>(logits, bias, T, E, k, o, idx, w, st);
  if (E <= 64) return launch_sg<LDT, 8, 8>(logits, bias, T, E, k, o, idx, w, st);
  if (E <= 128) return launch_sg<LDT, 16, 8>(logits, bias, T, E, k, o, idx, w, st);
  if (E <= 256) return launch_sg<LDT, 32, 8>(logits, bias, T, E, k, o, idx, w, st);
  if (E <= 512) return launch_sg<LDT, 64, 8>(logits, bias, T, E, k, o, idx, w, st);
  return launch_sg<LDT, 64, 16>(logits, bias, T, E, k, o, idx, w, st);
}

}  // namespace

hipError_t launch_route_sigmoid(const void* logits, int ldt, const float* bias,
                                int64_t T, int E, int k,
                                const GroupRouting& o, uint32_t* idx, void* w,
                                hipStream_t st) {
  switch (ldt) {
    case DT_F32: return launch_sigmoid_t<DT_F32>(logits, bias, T, E, k, o, idx, w, st);
    case DT_F16: return launch_sigmoid_t<DT_F16>(logits, bias, T, E, k, o, idx, w, st);
    default: return launch_sigmoid_t<DT_BF16>(logits, bias, T, E, k, o, idx, w, st);
  }
}

}  // namespace moe
