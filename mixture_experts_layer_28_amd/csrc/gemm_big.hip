// Large-tile segmented grouped GEMM for prefill-sized expert segments.
//
// Same operation and tile map as gemm.hip (docs.rs "ruDNN 0.1.25 source,
// src/moe/experts.rs", forward_dispatched_with_strategy: gate/up products
// with SiLU(gate)*up, then the down product), sized for MI355X:
//
// * 256 x 256 output tile per workgroup of 8 wavefronts in a 4 x 2 grid;
//   a wave owns 64 x 128 outputs as 4 x 8 v_mfma_f32_16x16x32 tiles with
//   FP32 accumulators, two waves per SIMD (one hides the other's LDS
//   latency).  The gate+up tile holds rows [n0, n0+128) of W_gate in B rows
//   0..127 and the same rows of W_up in 128..255; each wave takes matching
//   halves, so one lane holds g and u of the same output.
// * Operand tiles reach LDS without passing through registers: the buffer
//   unit writes LDS directly (buffer_load_dwordx4 ... lds, 16 bytes per
//   lane), one 1 KB block of 8 tile rows per instruction; each lane fetches
//   the global chunk that the row swizzle maps to its LDS slot.  Reads past
//   a segment's last row, a weight matrix's last row or K come back as
//   zeros (raw buffer range checks), so ragged tiles need no clamping; A
//   blocks wholly past the segment are not loaded and waves whose rows all
//   lie past it skip their MFMAs.
// * Two LDS stages of K = 64 (128 KB, one workgroup per CU) and one barrier
//   per stage; the loads of stage k+2 go out right after the barrier that
//   ends stage k, so they have a whole stage of MFMAs to land.
// * Measured on MI355X: this kernel is bound by operand delivery into the
//   CUs (global -> LDS), not by the MFMA or LDS-read rates.

#include "gemm_common.h"

namespace moe {
namespace {

constexpr int kBM = 256, kBK = 64;
template <int BN> constexpr int stage_elems() { return (kBM + BN) * kBK; }
template <int BN> constexpr size_t lds_bytes() { return 2 * stage_elems<BN>() * 2; }

template <int D, bool GATEUP, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_big_kernel(
    const typename Storage<D>::T* __restrict__ A,
    const typename Storage<D>::T* __restrict__ B0,
    const typename Storage<D>::T* __restrict__ B1,
    typename Storage<D>::T* __restrict__ C,
    const uint32_t* __restrict__ offsets, int64_t N, int K, int NB, int E,
    uint32_t ncol, int nseg) {
  using S = typename Storage<D>::T;
  using V = typename Frag<D>::V;
  constexpr int NT = 64 * WM * WN;
  constexpr int TM = kBM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int TCOLS = GATEUP ? BN / 2 : BN;
  constexpr int kStage = stage_elems<BN>();
  constexpr int NBLK = (kBM + BN) / 8;       // 1 KB LDS blocks per stage
  constexpr int BLK = NBLK / (WM * WN);       // ... per wave
  static_assert(NBLK % (WM * WN) == 0, "blocks per wave");
  static_assert(!GATEUP || FN % 2 == 0, "gate/up halves");
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  S* sm = (S*)smem_raw;
  __shared__ TileInfo ti;

  const int tid = threadIdx.x;
  if (tid < 64)
    locate_tile(blockIdx.x, gridDim.x, offsets, E, N, kBM, ncol, nseg, &ti);
  __syncthreads();
  if (!ti.found) return;
  const int e = uniform(ti.e);
  const int64_t hi = uniform(ti.hi), row0 = uniform(ti.row0);
  const int64_t n0 = (int64_t)uniform(ti.col) * TCOLS;

  if (e >= E) {  // rows of out-of-range experts: zeros
    for (int q = tid; q < kBM * TCOLS; q += NT) {
      const int64_t r = row0 + q / TCOLS, c = n0 + q % TCOLS;
      if (r < hi && c < NB) C[r * NB + c] = from_f32<D>(0.0f);
    }
    return;
  }

  const uint32_t rowbytes = (uint32_t)K * sizeof(S);
  // the A resource spans this tile's rows only, so every range fits in
  // 31 bits and OOB (2^31) is always past the end
  const int64_t arows = hi - row0 < kBM ? hi - row0 : kBM;
  const __amdgpu_buffer_rsrc_t rA =
      make_rsrc(A + row0 * K, (uint64_t)arows * rowbytes);
  const uint64_t wbytes = (uint64_t)NB * rowbytes;
  const __amdgpu_buffer_rsrc_t rB0 =
      make_rsrc(B0 + (int64_t)e * NB * K, wbytes);
  const __amdgpu_buffer_rsrc_t rB1 =
      GATEUP ? make_rsrc(B1 + (int64_t)e * NB * K, wbytes) : rB0;
  constexpr uint32_t OOB = 0x80000000u;

  const int wid = uniform(tid >> 6), lane = tid & 63;
  const int wm = wid / WN, wn = wid % WN;

  // ---- global -> LDS (direct) -------------------------------------------------
  // LDS stage: A rows 0..255 then B rows 0..BN-1, 128 bytes per row; block b
  // holds rows 8b..8b+7 of that sequence.
  auto dma = [&](int k0, int st) {
    S* base = sm + st * kStage;
#pragma unroll
    for (int j = 0; j < BLK; ++j) {
      const int b = wid + (WM * WN) * j;
      const int r = 8 * (b < 32 ? b : b - 32) + (lane >> 3);  // row within A or B
      const int c = (lane & 7) ^ swz(r);
      const int kk = k0 + c * 8;
      const bool kin = kk < K;
      if (b < 32) {
        // blocks wholly past the segment stay unloaded: only rows below
        // arows are ever stored, and the skip keeps a ragged tile's memory
        // traffic to its real rows (the uniform test costs no divergence)
        if (8 * b < arows)
          buffer_load_lds16(rA, base + b * 512,
                            kin ? (uint32_t)r * rowbytes + kk * (uint32_t)sizeof(S) : OOB);
      } else {
        const bool up = GATEUP && (b - 32) * 8 >= BN / 2;  // uniform
        const int br = up ? r - BN / 2 : r;
        buffer_load_lds16(up ? rB1 : rB0, base + b * 512,
                          kin ? (uint32_t)(n0 + br) * rowbytes + kk * (uint32_t)sizeof(S) : OOB);
      }
    }
  };

  // ---- fragments and MFMAs ----------------------------------------------------
  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A wave whose TM rows all lie past the segment (ragged last tile) has
  // nothing to compute; it still loads and meets the barriers.
  const bool active = wm * TM < arows;
  auto brow = [&](int j) -> int {
    if (GATEUP) {
      constexpr int H2 = FN / 2;
      return (j < H2 ? wn * (TN / 2) + j * 16
                     : BN / 2 + wn * (TN / 2) + (j - H2) * 16) +
             (lane & 15);
    }
    return wn * TN + j * 16 + (lane & 15);
  };
  auto read_frags = [&](int st, int half, V* fa, V* fb) {
    if (!active) return;
    const S* As = sm + st * kStage;
    const S* Bs = As + kBM * kBK;
    const int c = half * 4 + (lane >> 4);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = wm * TM + i * 16 + (lane & 15);
      fa[i] = *(const V*)&As[r * kBK + ((c ^ swz(r)) << 3)];
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int r = brow(j);
      fb[j] = *(const V*)&Bs[r * kBK + ((c ^ swz(r)) << 3)];
    }
  };
  auto mma = [&](const V* fa, const V* fb) {
    if (!active) return;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = Frag<D>::mma(fa[i], fb[j], acc[i][j]);
  };

  const int nk = (K + kBK - 1) / kBK;
  dma(0, 0);
  wait_vmem();
  __syncthreads();
  if (nk > 1) dma(kBK, 1);
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    V fa[FM], fb[FN];
    read_frags(st, 0, fa, fb);
    mma(fa, fb);
    read_frags(st, 1, fa, fb);
    mma(fa, fb);
    if (kt + 1 < nk) {
      wait_vmem();
      __syncthreads();  // stage kt+1 landed everywhere; stage kt fully read
      if (kt + 2 < nk) dma((kt + 2) * kBK, st);
    }
  }

  // ---- epilogue ---------------------------------------------------------------
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t r = row0 + wm * TM + i * 16 + (lane >> 4) * 4 + q;
      if (r >= hi) continue;
      S* crow = C + r * NB;
      if (GATEUP) {
        constexpr int H2 = FN / 2;
#pragma unroll
        for (int j = 0; j < H2; ++j) {
          const int64_t c = n0 + wn * (TN / 2) + j * 16 + (lane & 15);
          if (c < NB) {
            const float g = to_f32<D>(from_f32<D>(acc[i][j][q]));
            const float u = to_f32<D>(from_f32<D>(acc[i][j + H2][q]));
            crow[c] = from_f32<D>(silu_mul(g, u));
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int64_t c = n0 + wn * TN + j * 16 + (lane & 15);
          if (c < NB) crow[c] = from_f32<D>(acc[i][j][q]);
        }
      }
    }
  }
}

template <int D, bool GATEUP, int BN, int WM, int WN>
hipError_t launch_one(const void* A, const void* B0, const void* B1, void* C,
                      const uint32_t* offsets, int64_t N, int K, int NB,
                      int E, int nseg, hipStream_t st) {
  using S = typename Storage<D>::T;
  static bool attr = false;
  if (!attr) {
    hipError_t err = hipFuncSetAttribute(
        (const void*)gemm_big_kernel<D, GATEUP, BN, WM, WN>,
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes<BN>());
    if (err != hipSuccess) return err;
    attr = true;
  }
  const uint32_t ncol = cdiv(NB, GATEUP ? BN / 2 : BN);
  const uint32_t grid = tile_grid(ncol * (cdiv(N, kBM) + (uint32_t)nseg));
  hipLaunchKernelGGL((gemm_big_kernel<D, GATEUP, BN, WM, WN>), dim3(grid),
                     dim3(64 * WM * WN), lds_bytes<BN>(), st, (const S*)A,
                     (const S*)B0, (const S*)B1, (S*)C, offsets, N, K, NB, E,
                     ncol, nseg);
  return hipGetLastError();
}

template <int D>
hipError_t launch_pair(const void* xd, int64_t N, int64_t H, int64_t I,
                       int E, const void* wg, const void* wu, const void* wd,
                       const uint32_t* offsets, void* act, void* y,
                       hipStream_t st) {
  hipError_t err = launch_one<D, true, 256, 4, 2>(
      xd, wg, wu, act, offsets, N, (int)H, (int)I, E, E, st);
  if (err != hipSuccess) return err;
  timing_mark(5, st);
  return launch_one<D, false, 256, 4, 2>(act, wd, wd, y, offsets, N, (int)I,
                                         (int)H, E, E + 1, st);
}

}  // namespace

hipError_t launch_experts_big(const void* xd, int dt, int64_t N, int64_t H,
                              int64_t I, int E, const void* w_gate,
                              const void* w_up, const void* w_down,
                              const uint32_t* offsets, void* act, void* y,
                              hipStream_t st) {
  if (dt == DT_BF16)
    return launch_pair<DT_BF16>(xd, N, H, I, E, w_gate, w_up, w_down, offsets,
                                act, y, st);
  return launch_pair<DT_F16>(xd, N, H, I, E, w_gate, w_up, w_down, offsets,
                             act, y, st);
}

}  // namespace moe
