// Segmented grouped GEMMs of the SwiGLU experts.
//
// Source: docs.rs "ruDNN 0.1.25 source, src/moe/experts.rs".
// SwiGluExperts::new fixes bias-free gate/up weights [E,I,H] and down
// weights [E,H,I]; forward_dispatched_with_strategy computes, per expert
// segment of the dispatched rows, gate = X W_gate^T and up = X W_up^T (both
// "NT": every operand is contiguous along the reduction axis), overwrites
// gate with SiLU(gate) * up, and multiplies the result by W_down^T.
//
// Here the two first products share one kernel: a tile of output columns
// [n0, n0 + BN/2) loads BN/2 rows of W_gate and the same BN/2 rows of W_up,
// so every lane holds gate and up for the same (row, column) and applies
// SiLU(g) * u in the epilogue (g and u are rounded to the storage dtype
// first, as the reference stores them, then SiLU runs in FP32).  The down
// product is a second launch of the same kernel without the epilogue.
//
// Tiles: the grid covers an upper bound of the (expert, row block, column
// block) tiles, (ceil(N/BM) + segments) * column blocks, so no host sync is
// needed; each workgroup finds its tile from the device-side offsets (a
// prefix sum over the segments done by one wavefront) and exits if it has
// none.  Logical tile order is expert-major, then column block, then row
// block, so consecutive tiles share a weight tile; consecutive logical ids
// run on one XCD so they share that XCD's L2 (runs of 16 dealt round robin
// in the prefill and generic kernels, one contiguous range per XCD in the
// decode kernel, whose tiles are all alike).
//
// MFMA path (bf16/f16, K a multiple of 8, 16-byte aligned operands):
// 256 threads = 4 wavefronts in a WGM x (4/WGM) grid; v_mfma_f32_16x16x32
// (bf16 or f16) with FP32 accumulators; K steps of 64 staged through a
// double-buffered LDS tile whose 16-byte chunks are XOR-swizzled by row so
// the fragment reads (16 rows, one chunk) spread over the banks; the next
// K step's global loads are in flight while the current one is computed.
//
// Generic path (fp32, or shapes the MFMA path does not take): a 64x64 LDS
// tiled FMA kernel with element-wise bounds checks.
//
// A segment s = E (rows [offsets[E], N), produced by out-of-range expert
// ids) is written as zeros by the down launch.

#include "gemm_common.h"

#ifndef MOE_DECODE_NT
#define MOE_DECODE_NT true
#endif

namespace moe {
namespace {

// The plain tile map (BM-row blocks, locate_tile's logical order, one
// contiguous range of logical tiles per XCD), run by each wavefront on its own and broadcast to its
// lanes: the kernel then keeps no tile record in LDS and needs no barrier
// before its K loop, so four of its workgroups fit the 160 KB of LDS of a
// CU (the record pushed each one just past a quarter).
template <int BM>
__device__ inline TileInfo locate_tile_wave(uint32_t b,
                                            const uint32_t* __restrict__ offsets,
                                            int E, int64_t N,
                                            uint32_t ncol, int nseg) {
  const int lane = threadIdx.x & 63;
  TileInfo t;
  t.found = 0;
  t.e = t.col = t.rows = 0;
  t.lo = t.hi = t.row0 = 0;
  uint32_t total = 0;
  for (int s0 = 0; s0 < nseg; s0 += 64) {
    int64_t lo, hi;
    segment(offsets, s0 + lane, E, N, nseg, &lo, &hi);
    const uint32_t R32 = (uint32_t)(hi - lo);  // N < 2^32
    const uint32_t cnt = (R32 / BM + (R32 % BM != 0)) * ncol;
    total += __shfl(wave_inclusive_sum(cnt, lane), 63, 64);
  }
  const uint32_t per = (total + 7u) / 8u, local = b / 8u;
  const uint32_t L = (b % 8u) * per + local;
  if (local >= per || L >= total) return t;
  uint32_t base = 0;
  for (int s0 = 0; s0 < nseg; s0 += 64) {
    int64_t lo, hi;
    segment(offsets, s0 + lane, E, N, nseg, &lo, &hi);
    const uint32_t R32 = (uint32_t)(hi - lo);
    const uint32_t nt = R32 / BM + (R32 % BM != 0);
    const uint32_t cnt = nt * ncol;
    const uint32_t inc = wave_inclusive_sum(cnt, lane);
    const uint32_t exc = inc - cnt;
    const bool hit = L >= base + exc && L < base + inc;
    const uint64_t m = __ballot(hit);
    if (m) {
      const int src = (int)__builtin_ctzll(m);
      const int64_t slo = __shfl(lo, src, 64), shi = __shfl(hi, src, 64);
      const uint32_t snt = __shfl(nt, src, 64), sexc = __shfl(exc, src, 64);
      const uint32_t l = L - base - sexc;
      constexpr uint32_t GM = 8;
      const uint32_t grp = l / (GM * ncol), first = grp * GM;
      const uint32_t gs = snt - first < GM ? snt - first : GM;
      const uint32_t rem = l - grp * GM * ncol;
      t.e = s0 + src;
      t.lo = slo;
      t.hi = shi;
      t.col = (int)(rem / gs);
      t.row0 = slo + (int64_t)(first + rem % gs) * BM;
      t.rows = (int)(shi - t.row0 < BM ? shi - t.row0 : BM);
      t.found = 1;
      return t;
    }
    base += __shfl(inc, 63, 64);
  }
  return t;
}

template <int D, int BM, int BN, int WGM, bool GATEUP, bool NTW>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(
    const typename Storage<D>::T* __restrict__ A,
    const typename Storage<D>::T* __restrict__ B0,
    const typename Storage<D>::T* __restrict__ B1,
    typename Storage<D>::T* __restrict__ C,
    const uint32_t* __restrict__ offsets, int64_t N, int K, int NB, int E,
    uint32_t ncol, int nseg, Swiglu sw = Swiglu{}, Gather ga = Gather{}) {
  using S = typename Storage<D>::T;
  using V = typename Frag<D>::V;
  constexpr int BK = 64;
  constexpr int WGN = 4 / WGM;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int TCOLS = GATEUP ? BN / 2 : BN;  // output columns per tile
  constexpr int CA = BM * 8 / 256, CB = BN * 8 / 256;
  static_assert(CA >= 1 && CB >= 1 && FM >= 1 && FN >= (GATEUP ? 2 : 1), "tile");

  __shared__ __attribute__((aligned(16))) S As[2][BM * BK];
  __shared__ __attribute__((aligned(16))) S Bs[2][BN * BK];

  const int tid = threadIdx.x;
  const TileInfo ti =
      locate_tile_wave<BM>(blockIdx.x, offsets, E, N, ncol, nseg);
  if (!ti.found) return;  // the same answer in every wavefront
  const int e = uniform(ti.e);
  const int64_t hi = uniform(ti.hi), row0 = uniform(ti.row0);
  const int64_t n0 = (int64_t)uniform(ti.col) * TCOLS;

  if (e >= E) {  // rows of out-of-range experts: zeros
    for (int q = tid; q < BM * TCOLS; q += 256) {
      const int64_t r = row0 + q / TCOLS, c = n0 + q % TCOLS;
      if (r < hi && c < NB) C[r * NB + c] = from_f32<D>(0.0f);
    }
    return;
  }

  // global source of each 16-byte chunk this thread stages
  const S* pa[CA];
  const S* pb[CB];
  int ka[CA], kb[CB];
#pragma unroll
  for (int it = 0; it < CA; ++it) {
    const int q = tid + 256 * it, r = q >> 3, ch = q & 7;
    int64_t gr = row0 + r;
    gr = gr < hi ? gr : hi - 1;
    if (GATEUP && ga.rows) {  // the token row of x, clamped into x
      const int64_t tok = ga.rows[gr];
      gr = tok < ga.xrows ? tok : ga.xrows - 1;
    }
    pa[it] = A + gr * K + ch * 8;
    ka[it] = ch * 8;
  }
#pragma unroll
  for (int it = 0; it < CB; ++it) {
    const int q = tid + 256 * it, r = q >> 3, ch = q & 7;
    const S* base = B0;
    int64_t br = n0 + r;
    if (GATEUP && r >= BN / 2) {
      base = B1;
      br = n0 + r - BN / 2;
    }
    br = br < NB ? br : NB - 1;
    pb[it] = base + ((int64_t)e * NB + br) * K + ch * 8;
    kb[it] = ch * 8;
  }

  u32x4 ra[CA], rb[CB];
  auto load = [&](int k0) {
#pragma unroll
    for (int it = 0; it < CA; ++it)
      ra[it] = (k0 + ka[it] < K) ? *(const u32x4*)(pa[it] + k0) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int it = 0; it < CB; ++it) {
      const u32x4* src = (const u32x4*)(pb[it] + k0);
      rb[it] = (k0 + kb[it] < K) ? (NTW ? __builtin_nontemporal_load(src) : *src)
                                 : u32x4{0, 0, 0, 0};
    }
  };
  auto store = [&](int st) {
#pragma unroll
    for (int it = 0; it < CA; ++it) {
      const int q = tid + 256 * it, r = q >> 3, ch = q & 7;
      *(u32x4*)&As[st][r * BK + ((ch ^ swz(r)) << 3)] = ra[it];
    }
#pragma unroll
    for (int it = 0; it < CB; ++it) {
      const int q = tid + 256 * it, r = q >> 3, ch = q & 7;
      *(u32x4*)&Bs[st][r * BK + ((ch ^ swz(r)) << 3)] = rb[it];
    }
  };

  const int wid = tid >> 6, lane = tid & 63;
  const int wm = wid / WGN, wn = wid % WGN;
  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  int arow[FM], brow[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) arow[i] = wm * WTM + i * 16 + (lane & 15);
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    if (GATEUP) {
      constexpr int H2 = FN / 2;
      brow[j] = (j < H2 ? wn * (WTN / 2) + j * 16
                        : BN / 2 + wn * (WTN / 2) + (j - H2) * 16) +
                (lane & 15);
    } else {
      brow[j] = wn * WTN + j * 16 + (lane & 15);
    }
  }

  const int nk = (K + BK - 1) / BK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c = kk * 4 + (lane >> 4);
      V a[FM], b[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        a[i] = *(const V*)&As[st][arow[i] * BK + ((c ^ swz(arow[i])) << 3)];
#pragma unroll
      for (int j = 0; j < FN; ++j)
        b[j] = *(const V*)&Bs[st][brow[j] * BK + ((c ^ swz(brow[j])) << 3)];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = Frag<D>::mma(a[i], b[j], acc[i][j]);
    }
    if (kt + 1 < nk) store(st ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds rows 4*(lane/16)+i, column lane%16 of each fragment
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t r = row0 + wm * WTM + i * 16 + (lane >> 4) * 4 + q;
      if (r >= hi) continue;
      S* crow = C + r * NB;
      if (GATEUP) {
        constexpr int H2 = FN / 2;
#pragma unroll
        for (int j = 0; j < H2; ++j) {
          const int64_t c = n0 + wn * (WTN / 2) + j * 16 + (lane & 15);
          if (c < NB) {
            const float g = to_f32<D>(from_f32<D>(acc[i][j][q]));
            const float u = to_f32<D>(from_f32<D>(acc[i][j + H2][q]));
            crow[c] = from_f32<D>(swiglu_act(g, u, sw));
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int64_t c = n0 + wn * WTN + j * 16 + (lane & 15);
          if (c < NB) crow[c] = from_f32<D>(acc[i][j][q]);
        }
      }
    }
  }
}

// Generic FMA path: 64 x 64 tile (gate+up: 32 output columns), K step 16.
template <int D, bool GATEUP>
__global__ __launch_bounds__(256) void gemm_generic_kernel(
    const typename Storage<D>::T* __restrict__ A,
    const typename Storage<D>::T* __restrict__ B0,
    const typename Storage<D>::T* __restrict__ B1,
    typename Storage<D>::T* __restrict__ C,
    const uint32_t* __restrict__ offsets, int64_t N, int K, int NB, int E,
    uint32_t ncol, int nseg, Swiglu sw = Swiglu{}) {
  constexpr int BM = 64, BN = 64, BK = 16;
  constexpr int TCOLS = GATEUP ? 32 : 64;
  __shared__ float As[BK][BM + 1];
  __shared__ float Bs[BK][BN + 1];
  __shared__ TileInfo ti;
  const int tid = threadIdx.x;
  if (tid < 64)
    locate_tile<BM>(blockIdx.x, gridDim.x, offsets, E, N, ncol, nseg, &ti);
  __syncthreads();
  if (!ti.found) return;
  const int e = uniform(ti.e);
  const int64_t hi = uniform(ti.hi), row0 = uniform(ti.row0);
  const int64_t n0 = (int64_t)uniform(ti.col) * TCOLS;
  if (e >= E) {
    for (int q = tid; q < BM * TCOLS; q += 256) {
      const int64_t r = row0 + q / TCOLS, c = n0 + q % TCOLS;
      if (r < hi && c < NB) C[r * NB + c] = from_f32<D>(0.0f);
    }
    return;
  }
  const int ty = tid / 16, tx = tid % 16;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

  for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int q = tid + 256 * it, m = q / BK, kk = q % BK;
      int64_t gr = row0 + m;
      gr = gr < hi ? gr : hi - 1;
      As[kk][m] = (k0 + kk < K) ? to_f32<D>(A[gr * K + k0 + kk]) : 0.0f;
      int64_t br;
      const typename Storage<D>::T* base = B0;
      if (GATEUP) {
        br = n0 + (m < 32 ? m : m - 32);
        if (m >= 32) base = B1;
      } else {
        br = n0 + m;
      }
      br = br < NB ? br : NB - 1;
      Bs[kk][m] = (k0 + kk < K)
                      ? to_f32<D>(base[((int64_t)e * NB + br) * K + k0 + kk])
                      : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
      if (GATEUP) {
        b[0] = Bs[kk][tx * 2];
        b[1] = Bs[kk][tx * 2 + 1];
        b[2] = Bs[kk][32 + tx * 2];
        b[3] = Bs[kk][32 + tx * 2 + 1];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = row0 + ty * 4 + i;
    if (r >= hi) continue;
    if (GATEUP) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t c = n0 + tx * 2 + j;
        if (c < NB) {
          const float g = to_f32<D>(from_f32<D>(acc[i][j]));
          const float u = to_f32<D>(from_f32<D>(acc[i][j + 2]));
          C[r * NB + c] = from_f32<D>(swiglu_act(g, u, sw));
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t c = n0 + tx * 4 + j;
        if (c < NB) C[r * NB + c] = from_f32<D>(acc[i][j]);
      }
    }
  }
}

// NTW: every weight element is read by one tile only (decode-sized
// segments), so the weight tiles are streamed with nontemporal loads.
template <int D, int BM, int BN, int WGM, bool NTW>
hipError_t launch_mfma_pair(const void* xd, int64_t N, int64_t H, int64_t I,
                            int E, const void* wg, const void* wu,
                            const void* wd, const uint32_t* offsets,
                            void* act, void* y, hipStream_t st, Swiglu sw,
                            Gather ga = Gather{}) {
  using S = typename Storage<D>::T;
  {
    const uint32_t ncol = cdiv(I, BN / 2);
    const uint32_t grid = tile_grid(ncol * (cdiv(N, BM) + (uint32_t)E));
    hipLaunchKernelGGL((gemm_mfma_kernel<D, BM, BN, WGM, true, NTW>), dim3(grid),
                       dim3(256), 0, st, (const S*)xd, (const S*)wg,
                       (const S*)wu, (S*)act, offsets, N, (int)H, (int)I, E,
                       ncol, E, sw, ga);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  timing_mark(5, st);
  const uint32_t ncol = cdiv(H, BN);
  const uint32_t grid = tile_grid(ncol * (cdiv(N, BM) + (uint32_t)E + 1));
  hipLaunchKernelGGL((gemm_mfma_kernel<D, BM, BN, WGM, false, NTW>), dim3(grid),
                     dim3(256), 0, st, (const S*)act, (const S*)wd,
                     (const S*)wd, (S*)y, offsets, N, (int)I, (int)H, E,
                     ncol, E + 1);
  return hipGetLastError();
}

template <int D>
hipError_t launch_generic_pair(const void* xd, int64_t N, int64_t H,
                               int64_t I, int E, const void* wg,
                               const void* wu, const void* wd,
                               const uint32_t* offsets, void* act, void* y,
                               hipStream_t st, Swiglu sw) {
  using S = typename Storage<D>::T;
  {
    const uint32_t ncol = cdiv(I, 32);
    const uint32_t grid = tile_grid_chunked(ncol * (cdiv(N, 64) + (uint32_t)E));
    hipLaunchKernelGGL((gemm_generic_kernel<D, true>), dim3(grid), dim3(256),
                       0, st, (const S*)xd, (const S*)wg, (const S*)wu,
                       (S*)act, offsets, N, (int)H, (int)I, E, ncol, E, sw);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  timing_mark(5, st);
  const uint32_t ncol = cdiv(H, 64);
  const uint32_t grid = tile_grid_chunked(ncol * (cdiv(N, 64) + (uint32_t)E + 1));
  hipLaunchKernelGGL((gemm_generic_kernel<D, false>), dim3(grid), dim3(256),
                     0, st, (const S*)act, (const S*)wd, (const S*)wd,
                     (S*)y, offsets, N, (int)I, (int)H, E, ncol, E + 1);
  return hipGetLastError();
}

// Which MFMA kernels launch_mfma_dt takes: decode-sized 32-row tiles,
// the prefill kernel of gemm_big.hip (row blocks of up to 320 rows x 256
// columns, every buffer range under 2^31 bytes: the K-tail loads use offset
// 2^31 as "past the end", so a row block's A range, 320 rows of K
// elements, must stay below it), or 128 x 128 tiles.
enum class MfmaPath { kDecode, kBig, kMid };
MfmaPath mfma_path(int64_t N, int64_t H, int64_t I, int E) {
  if (N < 96 * (int64_t)E) return MfmaPath::kDecode;
  const int64_t lim = (int64_t)1 << 31;
  if (H * I * 2 < lim && 320 * H * 2 < lim && 320 * I * 2 < lim)
    return MfmaPath::kBig;
  return MfmaPath::kMid;
}

template <int D>
hipError_t launch_mfma_dt(const void* xd, int64_t N, int64_t H, int64_t I,
                          int E, const void* wg, const void* wu,
                          const void* wd, const uint32_t* offsets, void* act,
                          void* y, hipStream_t st, Swiglu sw, Gather ga) {
  switch (mfma_path(N, H, I, E)) {
    case MfmaPath::kDecode:  // few rows per expert: short row blocks
      return launch_mfma_pair<D, 32, 128, 1, MOE_DECODE_NT>(
          xd, N, H, I, E, wg, wu, wd, offsets, act, y, st, sw, ga);
    case MfmaPath::kBig:
      return launch_experts_big(xd, D, N, H, I, E, wg, wu, wd, offsets, act,
                                y, st, sw, ga);
    default:
      return launch_mfma_pair<D, 128, 128, 2, false>(
          xd, N, H, I, E, wg, wu, wd, offsets, act, y, st, sw, ga);
  }
}

// Plain grouped NT product on MFMA (bf16/f16, K and NB multiples of 8,
// 16-byte aligned): the kernels launch_experts would pick for its down GEMM.
template <int D>
hipError_t launch_nt_mfma(const void* A, int64_t N, int64_t K, const void* B,
                          int64_t NB, int E, const uint32_t* offsets, void* C,
                          hipStream_t st) {
  using S = typename Storage<D>::T;
  const int nseg = E + 1;  // rows past offsets[E] are written as zeros
  if (N < 96 * (int64_t)E) {
    const uint32_t ncol = cdiv(NB, 128);
    const uint32_t grid = tile_grid(ncol * (cdiv(N, 32) + (uint32_t)nseg));
    hipLaunchKernelGGL((gemm_mfma_kernel<D, 32, 128, 1, false, MOE_DECODE_NT>),
                       dim3(grid), dim3(256), 0, st, (const S*)A, (const S*)B,
                       (const S*)B, (S*)C, offsets, N, (int)K, (int)NB, E,
                       ncol, nseg);
    return hipGetLastError();
  }
  const int64_t lim = (int64_t)1 << 31;
  if (K * NB * 2 < lim && 320 * K * 2 < lim && 320 * NB * 2 < lim)
    return launch_nt_big(A, D, N, (int)K, B, (int)NB, E, offsets, C, st);
  const uint32_t ncol = cdiv(NB, 128);
  const uint32_t grid = tile_grid(ncol * (cdiv(N, 128) + (uint32_t)nseg));
  hipLaunchKernelGGL((gemm_mfma_kernel<D, 128, 128, 2, false, false>),
                     dim3(grid), dim3(256), 0, st, (const S*)A, (const S*)B,
                     (const S*)B, (S*)C, offsets, N, (int)K, (int)NB, E, ncol,
                     nseg);
  return hipGetLastError();
}

template <int D>
hipError_t launch_nt_generic(const void* A, int64_t N, int64_t K,
                             const void* B, int64_t NB, int E,
                             const uint32_t* offsets, void* C,
                             hipStream_t st) {
  using S = typename Storage<D>::T;
  const int nseg = E + 1;
  const uint32_t ncol = cdiv(NB, 64);
  const uint32_t grid = tile_grid_chunked(ncol * (cdiv(N, 64) + (uint32_t)nseg));
  hipLaunchKernelGGL((gemm_generic_kernel<D, false>), dim3(grid), dim3(256),
                     0, st, (const S*)A, (const S*)B, (const S*)B, (S*)C,
                     offsets, N, (int)K, (int)NB, E, ncol, nseg);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_nt(const void* A, int dt, int64_t N, int64_t K,
                             const void* B, int64_t NB, int E,
                             const uint32_t* offsets, void* C,
                             hipStream_t st) {
  const uintptr_t al = (uintptr_t)A | (uintptr_t)B | (uintptr_t)C;
  const bool mfma = dt != DT_F32 && K % 8 == 0 && NB % 8 == 0 && al % 16 == 0;
  if (mfma && dt == DT_BF16)
    return launch_nt_mfma<DT_BF16>(A, N, K, B, NB, E, offsets, C, st);
  if (mfma)
    return launch_nt_mfma<DT_F16>(A, N, K, B, NB, E, offsets, C, st);
  switch (dt) {
    case DT_F32: return launch_nt_generic<DT_F32>(A, N, K, B, NB, E, offsets, C, st);
    case DT_F16: return launch_nt_generic<DT_F16>(A, N, K, B, NB, E, offsets, C, st);
    default: return launch_nt_generic<DT_BF16>(A, N, K, B, NB, E, offsets, C, st);
  }
}

constexpr int64_t kGatherMaxColBlocks = 32;

bool experts_can_gather(int dt, int64_t N, int64_t H, int64_t I, int E,
                        int64_t xrows, const void* x, const void* w_gate,
                        const void* w_up, const void* w_down, const void* act,
                        const void* y) {
  const uintptr_t al = (uintptr_t)x | (uintptr_t)w_gate | (uintptr_t)w_up |
                       (uintptr_t)w_down | (uintptr_t)act | (uintptr_t)y;
  const bool mfma = dt != DT_F32 && H % 8 == 0 && I % 8 == 0 && al % 16 == 0;
  // The prefill kernel fetches each gathered A row slice once per column
  // block, each fetch behind an LDS read of the row's offset; with many
  // column blocks that costs more than the scatter it saves (Mixtral-shaped
  // layer, 112 gate+up column blocks: forward 3.4 % faster with the
  // scatter; fine-grained, 16 column blocks: the gather saves the 210 us
  // scatter).
  if (mfma && mfma_path(N, H, I, E) == MfmaPath::kBig &&
      2 * I > kGatherMaxColBlocks * 256)
    return false;
  // x is addressed by 32-bit byte offsets in the prefill kernel
  return mfma && xrows > 0 && xrows * H * 2 < ((int64_t)1 << 31);
}

hipError_t launch_experts(const void* xd, int dt, int64_t N, int64_t H,
                          int64_t I, int E, const void* w_gate,
                          const void* w_up, const void* w_down,
                          const uint32_t* offsets, void* act, void* y,
                          hipStream_t st, Swiglu sw, Gather ga) {
  const uintptr_t al = (uintptr_t)xd | (uintptr_t)w_gate | (uintptr_t)w_up |
                       (uintptr_t)w_down | (uintptr_t)act | (uintptr_t)y;
  const bool mfma = dt != DT_F32 && H % 8 == 0 && I % 8 == 0 && al % 16 == 0;
  if (mfma) {
    if (dt == DT_BF16)
      return launch_mfma_dt<DT_BF16>(xd, N, H, I, E, w_gate, w_up, w_down,
                                     offsets, act, y, st, sw, ga);
    return launch_mfma_dt<DT_F16>(xd, N, H, I, E, w_gate, w_up, w_down,
                                  offsets, act, y, st, sw, ga);
  }
  if (ga.rows) return hipErrorInvalidValue;  // callers check experts_can_gather
  switch (dt) {
    case DT_F32:
      return launch_generic_pair<DT_F32>(xd, N, H, I, E, w_gate, w_up, w_down,
                                         offsets, act, y, st, sw);
    case DT_F16:
      return launch_generic_pair<DT_F16>(xd, N, H, I, E, w_gate, w_up, w_down,
                                         offsets, act, y, st, sw);
    default:
      return launch_generic_pair<DT_BF16>(xd, N, H, I, E, w_gate, w_up,
                                          w_down, offsets, act, y, st, sw);
  }
}

}  // namespace moe
