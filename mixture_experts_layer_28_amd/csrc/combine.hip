// Combine kernel: weighted merge of the expert rows back into token order.
//
// Contract: ruDNN user guide (RUDA docs), section 6 "calling MoE": combine
// uses the dispatch mapping to restore token order and merges the expert
// outputs with the routing weights.  The weights are applied here only
// (section 12 states that the dispatch backward does not apply them again).
//
// out[t] = sum_{j<k} w[t,j] * y[token_row[t,j]], FP32 fused multiply-adds in
// slot order, rounded once to the activation dtype.  A workgroup takes a
// run of tokens; their k row ids and weights are staged in LDS, then the
// 256 threads stream 16-byte vectors of every row (HBM bound: N*H reads,
// T*H writes).  A row id >= N contributes NaN instead of being read.
//
// Without weights (a null pointer) every weight is 1, and the kernel is the
// dispatch backward of section 12: each token's selected rows summed in slot
// order (fmaf(1, v, acc) is the exact sum v + acc), rounded once.

#include "device_common.h"
#include "launch.h"

namespace moe {
namespace {

template <int D> struct Vec;  // 16-byte vectors of each storage type
template <> struct Vec<DT_F32> { static constexpr int n = 4; };
template <> struct Vec<DT_F16> { static constexpr int n = 8; };
template <> struct Vec<DT_BF16> { static constexpr int n = 8; };

// One output vector: slots in order; a row id >= N makes it NaN.  With KC
// (the top-k) known at compile time every slot's load is issued before
// the first multiply-add, so a thread has KC loads in flight.  NTL: y is
// far larger than the 256 MB Infinity Cache and is read with streaming
// loads (8192 x 7168, top-8: 203 us -> 191 us); a y that fits stays on
// ordinary loads, which find it in that cache after the down GEMM.
template <int D, int NV, int KC, bool NTL>
__device__ __forceinline__ void combine_vec(
    const typename Storage<D>::T* __restrict__ y, int64_t N, int64_t H,
    int k, const uint32_t* rows, const float* wts, int64_t v, float* acc) {
  using S = typename Storage<D>::T;
  constexpr int KN = KC > 0 ? KC : 1;
  const int kk = KC > 0 ? KC : k;
  for (int j0 = 0; j0 < kk; j0 += KN) {
    S vals[KN][NV];
#pragma unroll
    for (int j = 0; j < KN; ++j) {
      const uint32_t r = rows[j0 + j];
      if (r < (uint64_t)N) {
        if constexpr (NV * sizeof(S) == 16) {
          const u32x4* src = (const u32x4*)(y + (int64_t)r * H + v * NV);
          *(u32x4*)vals[j] = NTL ? __builtin_nontemporal_load(src) : *src;
        } else {
#pragma unroll
          for (int i = 0; i < NV; ++i) vals[j][i] = y[(int64_t)r * H + v * NV + i];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < KN; ++j) {
      const uint32_t r = rows[j0 + j];
      const float wt = wts[j0 + j];
      if (r < (uint64_t)N) {
#pragma unroll
        for (int i = 0; i < NV; ++i) acc[i] = fmaf(wt, to_f32<D>(vals[j][i]), acc[i]);
      } else {
#pragma unroll
        for (int i = 0; i < NV; ++i) acc[i] = __builtin_nanf("");
      }
    }
  }
}

template <int D, int WD, int NV, int KC, bool NTL>
__global__ __launch_bounds__(256) void combine_kernel(
    const typename Storage<D>::T* __restrict__ y, int64_t N, int64_t T,
    int64_t H, int k, const typename Storage<WD>::T* __restrict__ w,
    const uint32_t* __restrict__ token_row,
    typename Storage<D>::T* __restrict__ out, int tpb, int64_t vchunk) {
  using S = typename Storage<D>::T;
  extern __shared__ uint32_t sm[];
  uint32_t* srow = sm;
  float* sw = (float*)(sm + tpb * k);
  const int64_t t0 = (int64_t)blockIdx.x * tpb;
  for (int q = threadIdx.x; q < tpb * k; q += blockDim.x) {
    const int64_t t = t0 + q / k;
    if (t < T) {
      srow[q] = token_row[t0 * k + q];
      sw[q] = w ? to_f32<WD>(w[t0 * k + q]) : 1.0f;
    }
  }
  __syncthreads();
  const int64_t vpr = H / NV;  // vectors per row (NV elements each)
  // this block's vectors of each row: [v0, v0 + vlen) (blockIdx.y)
  const int64_t v0 = (int64_t)blockIdx.y * vchunk;
  const int64_t vlen = vpr - v0 < vchunk ? vpr - v0 : vchunk;
  const int64_t total = (int64_t)tpb * vlen;
  for (int64_t q = threadIdx.x; q < total; q += blockDim.x) {
    const int tl = (int)(q / vlen);
    const int64_t v = v0 + q - (int64_t)tl * vlen;
    const int64_t t = t0 + tl;
    if (t >= T) break;
    float acc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[i] = 0.0f;
    combine_vec<D, NV, KC, NTL>(y, N, H, k, srow + tl * k, sw + tl * k, v, acc);
    S res[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) res[i] = from_f32<D>(acc[i]);
    // the output is written once and not read back here: stream it
    if constexpr (NV * sizeof(S) == 16) {
      __builtin_nontemporal_store(*(const u32x4*)res, (u32x4*)(out + t * H + v * NV));
    } else {
#pragma unroll
      for (int i = 0; i < NV; ++i) out[t * H + v * NV + i] = res[i];
    }
  }
}

template <int D, int WD, int NV, bool NTL>
void launch_ck(const void* y, int64_t N, int64_t T, int64_t H, int k,
               const void* w, const uint32_t* token_row, void* out,
               dim3 grid, size_t lds, int tpb, int64_t vchunk,
               hipStream_t st) {
  using S = typename Storage<D>::T;
  using SW = typename Storage<WD>::T;
#define MOE_COMBINE(KC)                                                        \
  hipLaunchKernelGGL((combine_kernel<D, WD, NV, KC, NTL>), grid, dim3(256), lds, st, \
                     (const S*)y, N, T, H, k, (const SW*)w, token_row, (S*)out, \
                     tpb, vchunk)
  switch (k) {
    case 1: MOE_COMBINE(1); break;
    case 2: MOE_COMBINE(2); break;
    case 4: MOE_COMBINE(4); break;
    case 6: MOE_COMBINE(6); break;
    case 8: MOE_COMBINE(8); break;
    default: MOE_COMBINE(0); break;
  }
#undef MOE_COMBINE
}

template <int D, int WD>
hipError_t launch_c(const void* y, int64_t N, int64_t T, int64_t H, int k,
                    const void* w, const uint32_t* token_row, void* out,
                    hipStream_t st) {
  using S = typename Storage<D>::T;
  constexpr int NV = Vec<D>::n;
  if (T <= 0 || H <= 0) return hipSuccess;  // nothing to launch
  const bool vec_ok = H % NV == 0 && ((uintptr_t)y % 16 == 0) &&
                      ((uintptr_t)out % 16 == 0);
  const int64_t vpr = vec_ok ? H / NV : H;
  int64_t tpb = 1024 / vpr;
  if (tpb < 1) tpb = 1;
  if (tpb * k > 2048) tpb = 2048 / k;
  if (tpb < 1) tpb = 1;
  // Few token blocks (decode-sized batches): split each row's vectors over
  // grid.y so that about 256 workgroups share the loads, at least 64
  // vectors per row each, instead of a few workgroups walking whole rows.
  const int64_t nb = (T + tpb - 1) / tpb;
  int64_t nvc = 1;
  if (nb < 256) {
    nvc = (256 + nb - 1) / nb;
    const int64_t most = (vpr + 63) / 64;
    if (nvc > most) nvc = most;
    if (nvc < 1) nvc = 1;
  }
  const int64_t vchunk = (vpr + nvc - 1) / nvc;
  nvc = (vpr + vchunk - 1) / vchunk;
  const dim3 grid((unsigned)nb, (unsigned)nvc);
  const size_t lds = (size_t)tpb * k * 8;
  const bool stream = N * H * (int64_t)sizeof(S) > ((int64_t)128 << 20);
  if (vec_ok && stream)
    launch_ck<D, WD, NV, true>(y, N, T, H, k, w, token_row, out, grid, lds, (int)tpb, vchunk, st);
  else if (vec_ok)
    launch_ck<D, WD, NV, false>(y, N, T, H, k, w, token_row, out, grid, lds, (int)tpb, vchunk, st);
  else
    launch_ck<D, WD, 1, false>(y, N, T, H, k, w, token_row, out, grid, lds, (int)tpb, vchunk, st);
  (void)sizeof(S);
  return hipGetLastError();
}

template <int D>
hipError_t launch_cw(const void* y, int64_t N, int64_t T, int64_t H, int k,
                     const void* w, int wdt, const uint32_t* token_row,
                     void* out, hipStream_t st) {
  switch (wdt) {
    case DT_F32: return launch_c<D, DT_F32>(y, N, T, H, k, w, token_row, out, st);
    case DT_F16: return launch_c<D, DT_F16>(y, N, T, H, k, w, token_row, out, st);
    default: return launch_c<D, DT_BF16>(y, N, T, H, k, w, token_row, out, st);
  }
}

}  // namespace

hipError_t launch_combine(const void* y, int dt, int64_t N, int64_t T,
                          int64_t H, int k, const void* w, int wdt,
                          const uint32_t* token_row, void* out,
                          hipStream_t st) {
  switch (dt) {
    case DT_F32: return launch_cw<DT_F32>(y, N, T, H, k, w, wdt, token_row, out, st);
    case DT_F16: return launch_cw<DT_F16>(y, N, T, H, k, w, wdt, token_row, out, st);
    default: return launch_cw<DT_BF16>(y, N, T, H, k, w, wdt, token_row, out, st);
  }
}

}  // namespace moe
