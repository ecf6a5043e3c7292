// Router weights of a fixed selection and their logits gradient.
//
// Contract: ruDNN user guide (RUDA docs, German edition), section 12
// "first-order MoE training": selected_router_weights returns FP32 weights
// [T, top_k] for given indices; selected_router_backward returns the [T, E]
// logits gradient in the logits dtype for FP32 grad_weights.  Scores are the
// softmax over all E experts or the sigmoid of each logit; the selected
// scores are optionally renormalised by their sum, then multiplied by
// `scale`.  A repeated index gathers the same score again; an invalid index
// (negative, or >= E) makes the whole row NaN; only the continuous weights
// of the fixed selection are differentiated.
//
// With u_j the score of slot j's expert, g_j its incoming gradient,
// S = sum_l u_l, v_j = u_j / S and gbar = sum_l g_l v_l:
//   softmax:   dx_e = p_e * (A_e - sum_j u_j a_j),  a_j = scale * g_j
//   softmax, renormalised: the weights are the softmax over the selected
//              logits alone, so dx_e = sum of scale * v_j * (g_j - gbar)
//              over the slots selecting e, and 0 for the others (the form
//              without the two large terms that would cancel)
//   sigmoid:   dx_e = s_e * (1 - s_e) * A_e for a selected e, else exactly 0,
//              a_j = scale * g_j, or (scale / S) * (g_j - gbar) renormalised
// where A_e is the sum of a_j over the slots selecting e (a repeated index
// adds its slots).
// NaN propagates as the arithmetic carries it: under softmax a NaN, a +inf
// or an all -inf row makes every score NaN (the max subtraction); under
// sigmoid only the NaN logits' own scores are NaN.
//
// Layout: for E <= 1024 the softmax router's split, G lanes per row with
// PL = 8 (16 for E > 512) consecutive experts per lane in registers
// (router_weights_reg_kernel); wider rows take one wave per row walking the
// row in strides of 64 (router_weights_kernel).  The row's max and sum are
// butterfly reductions inside the group; the row's slots (top_k <= 64) are
// spread over the lanes, their expert ids and a_j go to LDS, and each lane
// then matches its experts against the slots.  Rows are walked in a
// grid-stride loop over a bounded grid.

#include "device_common.h"
#include "group_reduce.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kMaxSlots = 64;

__device__ __forceinline__ int64_t load_index(const void* ind, int it,
                                              int64_t i) {
  switch (it) {
    case IDX_U32: return (int64_t)((const uint32_t*)ind)[i];
    case IDX_I32: return (int64_t)((const int32_t*)ind)[i];
    default: return ((const int64_t*)ind)[i];
  }
}

// Register-cached form for E <= G * PL <= 1024, the lane split of the
// softmax router: lane l of a row's G lanes holds experts l*PL .. l*PL+PL-1
// (16-byte loads when VEC), the row's max and sum are group reductions of
// registers, the row is staged in LDS once for the slots' gathers, and each
// lane writes its PL gradient entries.  Several rows share a wave when
// G < 64, so far more rows are in flight than with a wave per row.
template <int LDT, int G, int PL, bool VEC, bool BWD>
__global__ __launch_bounds__(256) void router_weights_reg_kernel(
    const typename Storage<LDT>::T* __restrict__ logits, int64_t T, int E,
    const void* __restrict__ ind, int it, int k, int sigmoid, int renorm,
    float scale, const float* __restrict__ grad_w, float* __restrict__ w,
    typename Storage<LDT>::T* __restrict__ grad_x) {
  using S = typename Storage<LDT>::T;
  constexpr int R = 256 / G;                            // rows per pass
  constexpr int SS = G * PL < kMaxSlots ? G * PL : kMaxSlots;  // slots/row
  constexpr int SL = SS / G > 0 ? SS / G : 1;           // slots per lane
  __shared__ float xs[R * G * PL];
  __shared__ int sidx[R * SS];
  __shared__ float sa[R * SS];
  const int lane = threadIdx.x % G;
  const int xb = (int)(threadIdx.x / G) * G * PL;
  const int sb = (int)(threadIdx.x / G) * SS;
  const int e0 = lane * PL;

  for (int64_t base = (int64_t)blockIdx.x * R; base < T;
       base += (int64_t)gridDim.x * R) {
    const int64_t row = base + threadIdx.x / G;
    const bool live = row < T;
    const S* x = logits + row * (int64_t)E;

    float v[PL];
    if (live) {
      if constexpr (VEC) {
        constexpr int NE = 16 / sizeof(S);
        static_assert(PL % NE == 0, "whole vectors per lane");
#pragma unroll
        for (int q = 0; q < PL / NE; ++q) {
          S tmp[NE];
          *(u32x4*)tmp = *(const u32x4*)(x + e0 + q * NE);
#pragma unroll
          for (int i = 0; i < NE; ++i) v[q * NE + i] = to_f32<LDT>(tmp[i]);
        }
      } else {
#pragma unroll
        for (int m = 0; m < PL; ++m)
          v[m] = e0 + m < E ? to_f32<LDT>(x[e0 + m]) : 0.0f;
      }
    } else {
#pragma unroll
      for (int m = 0; m < PL; ++m) v[m] = 0.0f;
    }
#pragma unroll
    for (int m = 0; m < PL; ++m)
      if (e0 + m < E) xs[xb + e0 + m] = v[m];

    int bad = 0;
    if (live) {
      for (int j = lane; j < k; j += G) {
        const int64_t iv = load_index(ind, it, row * (int64_t)k + j);
        const bool ok = iv >= 0 && iv < E;
        sidx[sb + j] = ok ? (int)iv : -1;
        bad |= !ok;
      }
    }
    bad = group_or<G>(bad);

    float m = -INFINITY, sum = 0.0f;
    if (!sigmoid) {
#pragma unroll
      for (int q = 0; q < PL; ++q)
        if (e0 + q < E) m = fmaxf(m, v[q]);
      m = group_max<G>(m);
#pragma unroll
      for (int q = 0; q < PL; ++q)
        if (e0 + q < E) sum += expf(v[q] - m);
      sum = group_sum<G>(sum);
    }
    __syncthreads();

    float u[SL], gj[SL];
    float su = 0.0f, sgu = 0.0f;
#pragma unroll
    for (int q = 0; q < SL; ++q) {
      const int j = lane + G * q;
      u[q] = 0.0f;
      gj[q] = 0.0f;
      if (live && !bad && j < k) {
        const float xe = xs[xb + sidx[sb + j]];
        u[q] = sigmoid ? 1.0f / (1.0f + expf(-xe)) : expf(xe - m) / sum;
        su += u[q];
        if constexpr (BWD) {
          gj[q] = grad_w[row * (int64_t)k + j];
          sgu += gj[q] * u[q];
        }
      }
    }
    if (renorm) {
      su = group_sum<G>(su);
      if constexpr (BWD) sgu = group_sum<G>(sgu);
    }
    float dsum = 0.0f;
#pragma unroll
    for (int q = 0; q < SL; ++q) {
      const int j = lane + G * q;
      if (live && j < k) {
        if constexpr (BWD) {
          float a;
          if (!renorm) {
            a = scale * gj[q];
          } else {
            const float gbar = sgu / su;
            a = sigmoid ? (scale / su) * (gj[q] - gbar)
                        : scale * (u[q] / su) * (gj[q] - gbar);
          }
          sa[sb + j] = a;
          dsum += u[q] * a;
        } else {
          w[row * (int64_t)k + j] =
              bad ? __builtin_nanf("")
                  : (renorm ? scale * (u[q] / su) : scale * u[q]);
        }
      }
    }

    if constexpr (BWD) {
      if (!sigmoid && !renorm) dsum = group_sum<G>(dsum);
      __syncthreads();
      if (live) {
        S d[PL];
#pragma unroll
        for (int q = 0; q < PL; ++q) {
          const int e = e0 + q;
          float acc = 0.0f;
          bool hit = false;
          for (int j = 0; j < k; ++j) {
            if (sidx[sb + j] == e) {
              acc += sa[sb + j];
              hit = true;
            }
          }
          float dv;
          if (bad) {
            dv = __builtin_nanf("");
          } else if (sigmoid) {
            const float sv = 1.0f / (1.0f + expf(-v[q]));
            dv = hit ? sv * (1.0f - sv) * acc : 0.0f;
          } else if (renorm) {
            dv = hit ? acc : (expf(v[q] - m) / sum) * 0.0f;
          } else {
            dv = (expf(v[q] - m) / sum) * (acc - dsum);
          }
          d[q] = from_f32<LDT>(dv);
        }
        S* gx = grad_x + row * (int64_t)E + e0;
        if constexpr (VEC) {
          constexpr int NE = 16 / sizeof(S);
#pragma unroll
          for (int q = 0; q < PL / NE; ++q)
            *(u32x4*)(gx + q * NE) = *(const u32x4*)(d + q * NE);
        } else {
#pragma unroll
          for (int q = 0; q < PL; ++q)
            if (e0 + q < E) gx[q] = d[q];
        }
      }
    }
    __syncthreads();
  }
}

// Wide rows (E > 1024, or any E): G lanes per row walking the row in
// strides of G, the slots' logits re-read from memory.
template <int LDT, int G, bool BWD>
__global__ __launch_bounds__(256) void router_weights_kernel(
    const typename Storage<LDT>::T* __restrict__ logits, int64_t T, int E,
    const void* __restrict__ ind, int it, int k, int sigmoid, int renorm,
    float scale, const float* __restrict__ grad_w, float* __restrict__ w,
    typename Storage<LDT>::T* __restrict__ grad_x) {
  using S = typename Storage<LDT>::T;
  constexpr int R = 256 / G;
  __shared__ int sidx[R * kMaxSlots];
  __shared__ float sa[R * kMaxSlots];
  const int lane = threadIdx.x % G;
  const int rb = (int)(threadIdx.x / G) * kMaxSlots;

  for (int64_t base = (int64_t)blockIdx.x * R; base < T;
       base += (int64_t)gridDim.x * R) {
    const int64_t row = base + threadIdx.x / G;
    const bool live = row < T;
    const S* x = logits + row * (int64_t)E;

    // the row's expert ids; any invalid one poisons the row
    int bad = 0;
    if (live) {
      for (int j = lane; j < k; j += G) {
        const int64_t v = load_index(ind, it, row * (int64_t)k + j);
        const bool ok = v >= 0 && v < E;
        sidx[rb + j] = ok ? (int)v : -1;
        bad |= !ok;
      }
    }
    bad = group_or<G>(bad);

    // softmax max and sum over the whole row
    float m = -INFINITY, sum = 0.0f;
    if (!sigmoid) {
      if (live)
        for (int e = lane; e < E; e += G) m = fmaxf(m, to_f32<LDT>(x[e]));
      m = group_max<G>(m);
      if (live)
        for (int e = lane; e < E; e += G) sum += expf(to_f32<LDT>(x[e]) - m);
      sum = group_sum<G>(sum);
    }
    __syncthreads();

    // this lane's slots: scores, weights, and the slot terms a_j
    float u[kMaxSlots / 8], gj[kMaxSlots / 8];
    float su = 0.0f, sgu = 0.0f;
#pragma unroll
    for (int q = 0; q < kMaxSlots / 8; ++q) {
      const int j = lane + G * q;
      u[q] = 0.0f;
      gj[q] = 0.0f;
      if (live && !bad && j < k) {
        const float xe = to_f32<LDT>(x[sidx[rb + j]]);
        u[q] = sigmoid ? 1.0f / (1.0f + expf(-xe)) : expf(xe - m) / sum;
        su += u[q];
        if constexpr (BWD) {
          gj[q] = grad_w[row * (int64_t)k + j];
          sgu += gj[q] * u[q];
        }
      }
    }
    if (renorm) {
      su = group_sum<G>(su);
      if constexpr (BWD) sgu = group_sum<G>(sgu);
    }
    float dsum = 0.0f;  // sum_j u_j a_j
#pragma unroll
    for (int q = 0; q < kMaxSlots / 8; ++q) {
      const int j = lane + G * q;
      if (live && j < k) {
        if constexpr (BWD) {
          float a;
          if (!renorm) {
            a = scale * gj[q];
          } else {
            const float gbar = sgu / su;
            a = sigmoid ? (scale / su) * (gj[q] - gbar)
                        : scale * (u[q] / su) * (gj[q] - gbar);
          }
          sa[rb + j] = a;
          dsum += u[q] * a;
        } else {
          w[row * (int64_t)k + j] =
              bad ? __builtin_nanf("")
                  : (renorm ? scale * (u[q] / su) : scale * u[q]);
        }
      }
    }

    if constexpr (BWD) {
      if (!sigmoid && !renorm) dsum = group_sum<G>(dsum);
      __syncthreads();
      if (live) {
        S* gx = grad_x + row * (int64_t)E;
        for (int e = lane; e < E; e += G) {
          float acc = 0.0f;
          bool hit = false;
          for (int j = 0; j < k; ++j) {
            if (sidx[rb + j] == e) {
              acc += sa[rb + j];
              hit = true;
            }
          }
          float d;
          if (bad) {
            d = __builtin_nanf("");
          } else {
            const float xe = to_f32<LDT>(x[e]);
            if (sigmoid) {
              const float s = 1.0f / (1.0f + expf(-xe));
              d = hit ? s * (1.0f - s) * acc : 0.0f;
            } else if (renorm) {
              // 0 for an unselected logit, NaN if the row's scores are
              d = hit ? acc : (expf(xe - m) / sum) * 0.0f;
            } else {
              d = (expf(xe - m) / sum) * (acc - dsum);
            }
          }
          gx[e] = from_f32<LDT>(d);
        }
      }
    }
    // the next pass overwrites this pass's LDS rows
    __syncthreads();
  }
}

template <int LDT, int G, bool BWD>
hipError_t launch_rw_g(const void* logits, int64_t T, int E, const void* ind,
                       int it, int k, int sigmoid, int renorm, float scale,
                       const float* grad_w, float* w, void* grad_x,
                       hipStream_t st) {
  using S = typename Storage<LDT>::T;
  constexpr int R = 256 / G;
  const int64_t blocks = (T + R - 1) / R;
  const dim3 grid((unsigned)(blocks < 65536 ? blocks : 65536));
  hipLaunchKernelGGL((router_weights_kernel<LDT, G, BWD>), grid, dim3(256), 0,
                     st, (const S*)logits, T, E, ind, it, k, sigmoid, renorm,
                     scale, grad_w, w, (S*)grad_x);
  return hipGetLastError();
}

template <int LDT, int G, int PL, bool BWD>
hipError_t launch_rw_reg(const void* logits, int64_t T, int E,
                         const void* ind, int it, int k, int sigmoid,
                         int renorm, float scale, const float* grad_w,
                         float* w, void* grad_x, hipStream_t st) {
  using S = typename Storage<LDT>::T;
  constexpr int R = 256 / G;
  const int64_t blocks = (T + R - 1) / R;
  const dim3 grid((unsigned)(blocks < 65536 ? blocks : 65536));
  const bool vec = (PL * sizeof(S)) % 16 == 0 && E == G * PL &&
                   ((uintptr_t)logits | (uintptr_t)grad_x) % 16 == 0;
  if (vec)
    hipLaunchKernelGGL((router_weights_reg_kernel<LDT, G, PL, true, BWD>),
                       grid, dim3(256), 0, st, (const S*)logits, T, E, ind,
                       it, k, sigmoid, renorm, scale, grad_w, w, (S*)grad_x);
  else
    hipLaunchKernelGGL((router_weights_reg_kernel<LDT, G, PL, false, BWD>),
                       grid, dim3(256), 0, st, (const S*)logits, T, E, ind,
                       it, k, sigmoid, renorm, scale, grad_w, w, (S*)grad_x);
  return hipGetLastError();
}

template <int LDT, bool BWD>
hipError_t launch_rw_t(const void* logits, int64_t T, int E, const void* ind,
                       int it, int k, int sigmoid, int renorm, float scale,
                       const float* grad_w, float* w, void* grad_x,
                       hipStream_t st) {
#define MOE_RW_REG(G, PL)                                                    \
  return launch_rw_reg<LDT, G, PL, BWD>(logits, T, E, ind, it, k, sigmoid,   \
                                        renorm, scale, grad_w, w, grad_x, st)
  if (E <= 8) MOE_RW_REG(1, 8);
  if (E <= 16) MOE_RW_REG(2, 8);
  if (E <= 32) MOE_RW_REG(4, 8);
  if (E <= 64) MOE_RW_REG(8, 8);
  if (E <= 128) MOE_RW_REG(16, 8);
  if (E <= 256) MOE_RW_REG(32, 8);
  if (E <= 512) MOE_RW_REG(64, 8);
  if (E <= 1024) MOE_RW_REG(64, 16);
#undef MOE_RW_REG
  return launch_rw_g<LDT, 64, BWD>(logits, T, E, ind, it, k, sigmoid, renorm, scale, grad_w, w, grad_x, st);
}

template <bool BWD>
hipError_t launch_rw(const void* logits, int ldt, int64_t T, int E,
                     const void* ind, int it, int k, int sigmoid, int renorm,
                     float scale, const float* grad_w, float* w, void* grad_x,
                     hipStream_t st) {
  switch (ldt) {
    case DT_F32: return launch_rw_t<DT_F32, BWD>(logits, T, E, ind, it, k, sigmoid, renorm, scale, grad_w, w, grad_x, st);
    case DT_F16: return launch_rw_t<DT_F16, BWD>(logits, T, E, ind, it, k, sigmoid, renorm, scale, grad_w, w, grad_x, st);
    default: return launch_rw_t<DT_BF16, BWD>(logits, T, E, ind, it, k, sigmoid, renorm, scale, grad_w, w, grad_x, st);
  }
}

}  // namespace

hipError_t launch_selected_router_weights(const void* logits, int ldt,
                                          int64_t T, int E, const void* ind,
                                          int it, int k, int sigmoid,
                                          int renorm, float scale, float* w,
                                          hipStream_t st) {
  return launch_rw<false>(logits, ldt, T, E, ind, it, k, sigmoid, renorm,
                          scale, nullptr, w, nullptr, st);
}

hipError_t launch_selected_router_backward(const void* logits, int ldt,
                                           int64_t T, int E, const void* ind,
                                           int it, int k, const float* grad_w,
                                           int sigmoid, int renorm,
                                           float scale, void* grad_x,
                                           hipStream_t st) {
  return launch_rw<true>(logits, ldt, T, E, ind, it, k, sigmoid, renorm,
                         scale, grad_w, nullptr, grad_x, st);
}

}  // namespace moe
