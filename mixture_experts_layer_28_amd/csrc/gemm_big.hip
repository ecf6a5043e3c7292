// Large-tile segmented grouped GEMM for prefill-sized expert segments.
//
// Same operation and tile map as gemm.hip (docs.rs "ruDNN 0.1.25 source,
// src/moe/experts.rs", forward_dispatched_with_strategy: gate/up products
// with SiLU(gate)*up, then the down product), sized for MI355X:
//
// * Row blocks of up to 320 rows x 256 columns per workgroup of 8
//   wavefronts in a 4 x 2 grid.  A segment of R rows is cut into
//   ceil(R / 320) row blocks made of whole 32-row units dealt out evenly,
//   so a segment a few rows longer than a multiple of 256 does not leave a
//   thin last block that costs a whole pass over the weights, and no block
//   leaves a matrix-pipe slot of its busiest SIMD idle; a Mixtral-sized
//   segment of 1065 rows becomes blocks of 256, 288, 256 and 265 rows.  A
//   segment whose blocks would average more than 9 units is cut into
//   blocks of at most 8 units instead (kSplitUnits).  The 16-row MFMA row
//   tiles of a block are shared out over the 4 wave rows as evenly as
//   possible (at most 5 each); a wave owns up to 80 x 128 outputs as
//   v_mfma_f32_16x16x32 tiles with FP32 accumulators, two waves per SIMD.
//   The gate+up tile holds rows [n0, n0+128) of W_gate in B rows 0..127 and
//   the same rows of W_up in 128..255; each wave takes matching halves, so
//   one lane holds g and u of the same output.
// * Operand tiles reach LDS without passing through registers: the buffer
//   unit writes LDS directly (buffer_load_dwordx4 ... lds, 16 bytes per
//   lane), one 1 KB block of 8 tile rows per instruction; each lane fetches
//   the global chunk that the row swizzle maps to its LDS slot.  Reads past
//   a block's last row, a weight matrix's last row or K come back as zeros
//   (raw buffer range checks), so ragged tiles need no clamping; A blocks
//   wholly past the row block are not loaded.
// * Two LDS stages of K = 64 (2 x 72 KB, one workgroup per CU) and one
//   barrier per stage; the loads of stage k+2 go out right after the
//   barrier that ends stage k, so they have a whole stage of MFMAs to land.
//   The second half of a stage is multiplied after that barrier from
//   fragments read before it, while the next stage's first fragments are
//   read (a second register set for up to 4 row tiles, in-place reloads for
//   5), and the last stage is peeled so no branch merges those waits.
// * Measured on MI355X: the matrix pipes are busy 62-70 % of the active
//   cycles and the clock falls to 1.58-1.78 GHz under this load; the rest
//   is operand delivery into the CUs (global -> LDS) and the per-stage
//   barrier, not the MFMA or LDS-read rates (the LDS serves the fragment
//   reads about a quarter of the time).

#include "gemm_common.h"

#include <atomic>
#include <type_traits>

namespace moe {
namespace {

constexpr int kBM = 320, kBN = 256, kBK = 64;
// Segments whose 320-row blocks would average more than kSplitUnits units
// of 32 rows are cut into blocks of at most 256 rows (locate_tile's
// `split`): blocks of 288-320 rows give every wave row five MFMA row tiles,
// whose K loop cannot hold a second fragment set, and the skewed
// fine-grained routing made 76 % of its blocks so.  Measured in a
// same-process A/B at that shape: the down GEMM ~5 % faster and the
// forward 2.2 %; the Mixtral shape (blocks of 256-288 rows) unchanged.
// The gate+up product reading token rows in place keeps 320-row blocks
// (with the split that launch was 2-4 % slower).
constexpr int kSplitUnits = 9;
// Weight-gradient tiles per XCD chunk (see the weight-gradient form below).
constexpr uint32_t kWgChunk = 4;
// Weight-gradient tiles: kWgBM x kBN outputs; K-major stage parts of 16
// groups of 4 K rows, each group 4 x 256 elements + 32 of padding.
constexpr int kWgBM = 256;
constexpr int kWgGroup = 4 * 256 + 32;
constexpr int kWgPart = 16 * kWgGroup;
constexpr int kFM = kBM / 4 / 16;                 // MFMA row tiles per wave, at most
constexpr int kStage = (kBM + kBN) * kBK;         // elements of one LDS stage
constexpr size_t kLds = 2 * kStage * 2;           // two stages of 16-bit data
static_assert(2 * kWgPart <= kStage, "both K-major parts fit a stage");

// Opt a kernel in to kLds bytes of dynamic LDS, once per device (the
// attribute belongs to each device's copy of the kernel); `done` holds one
// bit per device id below 64, set once the call succeeded there.
inline hipError_t allow_lds(const void* fn, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  const uint64_t bit = dev >= 0 && dev < 64 ? (1ull << dev) : 0ull;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)kLds);
  if (err == hipSuccess) done.fetch_or(bit, std::memory_order_release);
  return err;
}

// ---- tiles of at most kTinyRows rows ---------------------------------------
// A row block this short has almost no MFMA work: its cost is streaming the
// 256 weight rows of its column block over the whole K.  Such a tile keeps
// three LDS stages of (kTinyRows + 256) rows x 64 K in flight instead of
// the main loop's two stages of up to 576 rows, so its loads go out two
// stages ahead of their use, and every wave computes all the tile's row
// tiles for 32 of its 256 columns (gate+up: 16 act columns, gate and up).
// (A non-inlined call cost the main loop SGPR spills; inlined, the
// fine-grained forward runs ~1 % faster and the Mixtral-shaped one is
// unchanged.)
constexpr int kTinyRows = 64;
constexpr int kTinyStage = (kTinyRows + kBN) * kBK;  // elements per stage
constexpr int kTinyStages = 3;
static_assert(kTinyStages * kTinyStage * 2 <= (int)kLds, "tiny stages fit");

// A raw buffer resource from a pointer and size every lane agrees on.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_u(const void* p,
                                                            uint64_t bytes) {
  const uint64_t u = (uint64_t)uniform((int64_t)(uintptr_t)p);
  return make_rsrc((const void*)(uintptr_t)u, (uint64_t)uniform((int64_t)bytes));
}

template <int D, bool GATEUP, bool GATHER, bool CLIP>
__device__ __forceinline__ void tiny_tile(
    const typename Storage<D>::T* A, const typename Storage<D>::T* B0,
    const typename Storage<D>::T* B1, typename Storage<D>::T* C,
    const uint32_t* grows, int64_t xrows, int64_t row0, int arows,
    int64_t n0, int e, int K, int NB, Swiglu sw) {
  using S = typename Storage<D>::T;
  using V = typename Frag<D>::V;
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  S* sm = (S*)smem_raw;
  constexpr uint32_t OOB = 0x80000000u;
  row0 = uniform(row0);
  arows = uniform(arows);
  n0 = uniform(n0);
  e = uniform(e);
  K = uniform(K);
  NB = uniform(NB);
  const uint32_t rowbytes = (uint32_t)K * sizeof(S);
  const __amdgpu_buffer_rsrc_t rA =
      GATHER ? make_rsrc_u(A, (uint64_t)xrows * rowbytes)
             : make_rsrc_u(A + row0 * K, (uint64_t)arows * rowbytes);
  const __amdgpu_buffer_rsrc_t rB0 =
      make_rsrc_u(B0 + (int64_t)e * NB * K, (uint64_t)NB * rowbytes);
  const __amdgpu_buffer_rsrc_t rB1 =
      GATEUP ? make_rsrc_u(B1 + (int64_t)e * NB * K, (uint64_t)NB * rowbytes)
             : rB0;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = uniform(tid >> 6);
  // this lane's A row (its wave's one A block) and its byte offset
  const int ar = 8 * wid + (lane >> 3);
  uint32_t aoff = OOB;
  if (ar < arows) {
    if (GATHER) {
      const uint32_t tok = grows[row0 + ar];
      if ((int64_t)tok < xrows) aoff = tok * rowbytes;
    } else {
      aoff = (uint32_t)ar * rowbytes;
    }
  }
  // every wave issues exactly 5 loads per stage (one A block, four B
  // blocks; A rows past the tile read zeros), so vmcnt counts stages
  auto dma = [&](int k0, int st) {
    S* base = sm + st * kTinyStage;
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const int b = wid + 8 * j;
      const int r = 8 * (j == 0 ? b : b - 8) + (lane >> 3);
      const int kk = k0 + ((lane & 7) ^ swz(r)) * 8;
      const bool kin = kk < K;
      if (j == 0) {
        buffer_load_lds16(rA, base + b * 512,
                          kin && aoff != OOB ? aoff + kk * (uint32_t)sizeof(S) : OOB);
      } else {
        const bool up = GATEUP && r >= kBN / 2;  // uniform per block
        const int br = up ? r - kBN / 2 : r;
        buffer_load_lds16(up ? rB1 : rB0, base + b * 512,
                          kin ? (uint32_t)(n0 + br) * rowbytes + kk * (uint32_t)sizeof(S) : OOB);
      }
    }
  };
  const int t16 = (arows + 15) >> 4;  // 1 .. 4 row tiles, all in every wave
  // B rows of this wave's two column tiles
  const int b0 = GATEUP ? wid * 16 : wid * 32;
  const int b1 = GATEUP ? kBN / 2 + wid * 16 : wid * 32 + 16;
  f32x4 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nk = (K + kBK - 1) / kBK;
  dma(0, 0);
  if (nk > 1) dma(kBK, 1);
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt landed everywhere; everyone finished reading stage kt - 1
    if (kt + 1 < nk)
      asm volatile("s_waitcnt vmcnt(5)\n\ts_barrier" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if (kt + 2 < nk) dma((kt + 2) * kBK, (kt + 2) % kTinyStages);
    const S* As = sm + (kt % kTinyStages) * kTinyStage;
    const S* Bs = As + kTinyRows * kBK;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int c = half * 4 + (lane >> 4);
      const int r0 = b0 + (lane & 15), r1 = b1 + (lane & 15);
      const V fb0 = *(const V*)&Bs[r0 * kBK + ((c ^ swz(r0)) << 3)];
      const V fb1 = *(const V*)&Bs[r1 * kBK + ((c ^ swz(r1)) << 3)];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < t16) {
          const int r = i * 16 + (lane & 15);
          const V fa = *(const V*)&As[r * kBK + ((c ^ swz(r)) << 3)];
          acc[i][0] = Frag<D>::mma(fa, fb0, acc[i][0]);
          acc[i][1] = Frag<D>::mma(fa, fb1, acc[i][1]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i >= t16) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rr = i * 16 + (lane >> 4) * 4 + q;
      if (rr >= arows) continue;
      S* crow = C + (row0 + rr) * NB;
      if (GATEUP) {
        const int64_t c = n0 + wid * 16 + (lane & 15);
        if (c < NB) {
          const float g = to_f32<D>(from_f32<D>(acc[i][0][q]));
          const float u = to_f32<D>(from_f32<D>(acc[i][1][q]));
          crow[c] = from_f32<D>(swiglu_act_t<CLIP>(g, u, sw));
        }
      } else {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int64_t c = n0 + wid * 32 + jj * 16 + (lane & 15);
          if (c < NB) crow[c] = from_f32<D>(acc[i][jj][q]);
        }
      }
    }
  }
}

// WG: the weight-gradient form.  Per expert e with rows [lo, hi) of a
// dispatch, Cw[e] [M, NB] (FP32) = A_e^T . B_e with A_e = rows lo .. hi-1 of
// A [N, M] and B_e = the same rows of B0 [N, NB]: both operands are read in
// place, K-major (K = hi - lo, the expert's row count), into LDS groups of
// 4 K rows and out of LDS with transposing reads (no per-expert transposed
// copies).  The tiles are E x ceil(M / kWgBM) x ncol (row blocks of whole
// 16-row units), dealt to the XCDs in chunks of kWgChunk tiles, round
// robin.  A tile's cost grows with its expert's rows: contiguous ranges of
// equal tile counts per XCD gave the XCD holding the largest experts of a
// skewed routing about 1.5 times the mean work (the fine-grained expert
// backward ran 19 % faster with chunks of 4; chunks of 2, 8, 16, 32 and 64
// measured 17.3, 17.3, 17.8, 17.8 and 18.6 ms against 17.2, and the
// balanced Mixtral-shaped backward stayed within 1 %).  An expert without
// rows writes zeros.  N is the row count of the dispatch, M passes in `K`.
// GATHER (gate+up only): A row r of the segments is row ga.rows[r] of the
// token rows x = A [ga.xrows, K] instead of row r of the dispatched copy.
// ALT: with GATEUP, the clipped SwiGLU activation; on a plain product, the
// NN form: B is stored K-major ([E, K, NB], e.g. a weight tensor used
// untransposed) and read through the LDS's transposing reads.
template <int D, bool GATEUP, bool WG = false, bool GATHER = false,
          bool ALT = false>
__global__ __launch_bounds__(512, 1) void gemm_big_kernel(
    const typename Storage<D>::T* __restrict__ A,
    const typename Storage<D>::T* __restrict__ B0,
    const typename Storage<D>::T* __restrict__ B1,
    typename Storage<D>::T* __restrict__ C,
    const uint32_t* __restrict__ offsets, int64_t N, int K, int NB, int E,
    uint32_t ncol, int nseg, float* __restrict__ Cw = nullptr,
    Swiglu sw = Swiglu{}, Gather ga = Gather{}, int split = 0) {
  using S = typename Storage<D>::T;
  using V = typename Frag<D>::V;
  constexpr bool CLIP = GATEUP && ALT;
  constexpr bool NN = !GATEUP && !WG && ALT;
  constexpr int WN = 2, NT = 512;
  constexpr int TN = kBN / WN;                    // 128 columns per wave
  constexpr int FN = TN / 16;                     // 8 MFMA column tiles
  constexpr int TCOLS = GATEUP ? kBN / 2 : kBN;
  constexpr int NBLK = (kBM + kBN) / 8;           // 1 KB LDS blocks per stage
  constexpr int ABLK = kBM / 8;
  constexpr int BLK = WG ? 8 : NBLK / 8;          // ... per wave
  static_assert(NBLK % 8 == 0, "blocks per wave");
  static_assert(!GATEUP || FN % 2 == 0, "gate/up halves");
  static_assert(FN == 8, "an 8-column group per lane: one 16-byte vector");
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  S* sm = (S*)smem_raw;
  __shared__ TileInfo ti;
  // GATHER: byte offset in x of each A row of the block (rows past it: OOB)
  __shared__ uint32_t arow_off[GATHER ? kBM : 1];

  const int tid = threadIdx.x;
  const int64_t Mw = K;  // the weight-gradient form's M (rows of Cw[e])
  int e, arows;
  int64_t row0, n0;
  const S* Ab = A;
  const S* Bb = B0;
  if constexpr (WG) {
    // static map: tile L -> (expert, row block, column block)
    const int64_t M = K;
    const uint32_t nmb = (uint32_t)((M + kWgBM - 1) / kWgBM);
    const uint32_t total = (uint32_t)E * nmb * ncol;
    const uint32_t local = blockIdx.x / 8u, q = local / kWgChunk;
    const uint32_t L =
        (q * 8u + blockIdx.x % 8u) * kWgChunk + local % kWgChunk;
    if (L >= total) return;
    e = (int)(L / (nmb * ncol));
    const uint32_t l = L % (nmb * ncol);
    const uint32_t grp = l / (8u * ncol), first = grp * 8u;
    const uint32_t gs = nmb - first < 8u ? nmb - first : 8u;
    const uint32_t rem = l - grp * 8u * ncol;
    const int64_t mb = first + rem % gs;
    n0 = (int64_t)(rem / gs) * TCOLS;
    // row blocks of whole 16-row units: every block starts 32-byte aligned
    // in a K-major row, so no 16-byte operand chunk straddles a buffer end
    const int64_t u16 = (M + 15) / 16;
    const int64_t a = 16 * (mb * u16 / nmb);
    const int64_t z0 = 16 * ((mb + 1) * u16 / nmb), z = z0 < M ? z0 : M;
    row0 = a;
    arows = (int)(z - a);
    int64_t hi = uniform((int64_t)offsets[e + 1]);
    hi = hi < N ? hi : N;
    int64_t lo = uniform((int64_t)offsets[e]);
    lo = lo < hi ? lo : hi;
    K = (int)(hi - lo);
    Ab = A + lo * M;
    Bb = B0 + lo * (int64_t)NB;
    if (K == 0) {  // no rows: a zero gradient
      float* ce = Cw + (int64_t)e * M * NB;
      for (int q = tid; q < kBM * TCOLS; q += NT) {
        const int64_t r = row0 + q / TCOLS, c = n0 + q % TCOLS;
        if (r < row0 + arows && c < NB) ce[r * NB + c] = 0.0f;
      }
      return;
    }
  } else {
    if (tid < 64)
      locate_tile<kBM>(blockIdx.x, gridDim.x, offsets, E, N, ncol, nseg, &ti,
                       true, split);
    __syncthreads();
    if (!ti.found) return;
    e = uniform(ti.e);
    row0 = uniform(ti.row0);
    arows = uniform(ti.rows);                     // 1 .. kBM
    n0 = (int64_t)uniform(ti.col) * TCOLS;
  }
  const int64_t tend = row0 + arows;

  if (!WG && e >= E) {  // rows of out-of-range experts: zeros
    for (int q = tid; q < kBM * TCOLS; q += NT) {
      const int64_t r = row0 + q / TCOLS, c = n0 + q % TCOLS;
      if (r < tend && c < NB) C[r * NB + c] = from_f32<D>(0.0f);
    }
    return;
  }
  if (!WG && !NN && arows <= kTinyRows) {
    tiny_tile<D, GATEUP, GATHER, CLIP>(A, B0, B1, C, ga.rows, ga.xrows, row0,
                                 arows, n0, e, K, NB, sw);
    return;
  }

  constexpr uint32_t OOB = 0x80000000u;
  const uint32_t rowbytes = (uint32_t)K * sizeof(S);
  // the A resource spans this tile's rows only (or, gathering, the token
  // rows x [xrows, K], under 2^31 bytes; in the weight-gradient form, the
  // expert's rows of the K-major operands), so every range fits in 31 bits
  // and OOB (2^31) is always past the end
  const __amdgpu_buffer_rsrc_t rA =
      WG       ? make_rsrc(Ab, (uint64_t)K * (uint64_t)Mw * sizeof(S))
      : GATHER ? make_rsrc(A, (uint64_t)ga.xrows * rowbytes)
               : make_rsrc(Ab + row0 * K, (uint64_t)arows * rowbytes);
  const __amdgpu_buffer_rsrc_t rB0 =
      WG ? make_rsrc(Bb, (uint64_t)K * (uint64_t)NB * sizeof(S))
         : make_rsrc(B0 + (int64_t)e * NB * K, (uint64_t)NB * rowbytes);
  const __amdgpu_buffer_rsrc_t rB1 =
      GATEUP ? make_rsrc(B1 + (int64_t)e * NB * K, (uint64_t)NB * rowbytes)
             : rB0;
  const int64_t boff = n0;  // B row of the tile's first column

  const int wid = uniform(tid >> 6) & 7, lane = tid & 63;
  const int wm = wid / WN, wn = wid % WN;
  // B rows in LDS, permuted so that each lane's MFMA columns are
  // consecutive output columns while every fragment read still covers
  // consecutive LDS rows (their chunks rotate by LDS row like A's).  Plain
  // products: a lane's 8 columns are 8 consecutive outputs, so B row
  // r = 64a + 8b + c is kept at LDS row 64a + 8c + b (rotating rows 8
  // apart by row / 8 instead left bank conflicts).  Gate+up: a lane's 4
  // gate columns, and the 4 up columns paired with them, are 4 consecutive
  // act columns, so gate (or up) row r = 64a + 4n + j is kept at LDS row
  // 64a + 16j + n.
  auto bsrc = [](int R) {  // B tile row held at LDS row R
    return GATEUP ? (R & ~63) | ((R & 15) << 2) | ((R >> 4) & 3)
                  : (R & ~63) | ((R & 7) << 3) | ((R >> 3) & 7);
  };

  // MFMA row tiles of this wave: t16 tiles over 4 wave rows, the first
  // t16 % 4 rows taking one more; waves wm and wm + 2 share a SIMD.
  const int t16 = (arows + 15) >> 4;
  const int fm = (t16 >> 2) + (wm < (t16 & 3) ? 1 : 0);
  const int tr0 = 16 * (wm * (t16 >> 2) + (wm < (t16 & 3) ? wm : (t16 & 3)));

  // ---- global -> LDS (direct) -------------------------------------------------
  // LDS stage: A rows 0..kBM-1 then B rows 0..255, 128 bytes per row; block
  // b holds rows 8b..8b+7 of that sequence.  Gathering, A row r sits at
  // the byte offset arow_off[r] of x (its token's row; rows past the block
  // read zeros).
  if constexpr (GATHER) {
    for (int q = tid; q < kBM; q += NT) {
      uint32_t off = OOB;
      if (q < arows) {
        const uint32_t tok = ga.rows[row0 + q];
        if ((int64_t)tok < ga.xrows) off = tok * rowbytes;
      }
      arow_off[q] = off;
    }
    __syncthreads();
  }
  auto dma = [&](int k0, int st) {
    S* base = sm + st * kStage;
    if constexpr (WG) {
      // K-major operands, 4 K rows at a time: the A part (then the B part)
      // of a stage holds, per group q of 4 K rows, 16 slots of 16 columns
      // (64 bytes each row, the 4 rows one after another) and 64 bytes of
      // padding: 16-byte chunk w of a group is slot w / 8, row (w / 2) % 4,
      // columns 8 (w % 2) .. + 7 of the slot.  The padding puts groups 2
      // apart (the ones a transposing read takes for lanes 0-15 and 16-31)
      // on different halves of the 256-byte bank cycle.  Each wave loads
      // 4 A and 4 B blocks of 1 KB (half a group); chunks past K or past
      // the matrix read zeros.
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int b = wid + 8 * (j & 3), q = b >> 1, w = 64 * (b & 1) + lane;
        const int k = k0 + 4 * q + ((w >> 1) & 3);
        const int c = 16 * (w >> 3) + 8 * (w & 1);
        S* dst = base + (j < 4 ? 0 : kWgPart) + q * kWgGroup + 512 * (b & 1);
        if (j < 4) {
          const int m = (int)row0 + c;
          const uint32_t o =
              k < K && m < Mw
                  ? ((uint32_t)k * (uint32_t)Mw + (uint32_t)m) * sizeof(S)
                  : OOB;
          buffer_load_lds16(rA, dst, o);
        } else {
          const int n = (int)n0 + c;
          uint32_t o =
              k < K && n < NB
                  ? ((uint32_t)k * (uint32_t)NB + (uint32_t)n) * sizeof(S)
                  : OOB;
          asm volatile("" : "+v"(o));
          buffer_load_lds16(rB0, dst, o);
        }
      }
      return;
    }
    // branch-free: which slots hold A or B blocks, and which B rows are
    // up rows, is fixed per unrolled slot (wid < 8), so the issue is
    // straight-line code (it was a chain of uniform branches per block)
    constexpr int AJ = ABLK / 8;  // A blocks per wave: wave w takes w + 8 j
    // Gathering: the wave's A row offsets, read together (one LDS round
    // trip before the loads instead of one per load; volatile so the
    // compiler keeps them out of registers between K steps: held there they
    // spilled).  The pointer keeps the LDS address space: a volatile read
    // through a generic pointer is a flat load with the coherence bits set,
    // which waits on the vector-memory counter too and holds a 64-bit
    // address per read (fine-grained forward 3 % faster as LDS reads).
    uint32_t ao[AJ];
    if constexpr (GATHER) {
      typedef volatile __attribute__((address_space(3))) uint32_t lds_u32;
#pragma unroll
      for (int j = 0; j < AJ; ++j)
        ao[j] = ((lds_u32*)arow_off)[8 * (wid + 8 * j) + (lane >> 3)];
    }
#pragma unroll
    for (int j = 0; j < BLK; ++j) {
      if (j < AJ) {
        const int b = wid + 8 * j;  // A block; rows past the tile read zeros
        const int r = 8 * b + (lane >> 3);
        const int kk = k0 + ((lane & 7) ^ swz(r)) * 8;
        const uint32_t ro = GATHER ? ao[j] : (uint32_t)r * rowbytes;
        buffer_load_lds16(rA, base + b * 512,
                          kk < K ? ro + kk * (uint32_t)sizeof(S) : OOB);
      } else if constexpr (NN) {
        // K-major B: group q of 4 K rows holds 16 slots of 16 columns (the
        // 4 rows' 16 columns one after another, 128 bytes); slot t holds
        // columns 16 (t ^ ((q / 2) % 2)) .. + 15, which puts the two groups
        // a transposing read takes for lanes 0-15 and 16-31 on different
        // halves of the 256-byte bank cycle
        const int bb = wid + 8 * (j - AJ);  // B block: half a group
        const int q = bb >> 1, w = 64 * (bb & 1) + lane;
        const int n =
            (int)n0 + 16 * ((w >> 3) ^ ((q >> 1) & 1)) + 8 * (w & 1);
        const int k = k0 + 4 * q + ((w >> 1) & 3);
        uint32_t bo =
            k < K && n < NB
                ? ((uint32_t)k * (uint32_t)NB + (uint32_t)n) * sizeof(S)
                : OOB;
        asm volatile("" : "+v"(bo));
        buffer_load_lds16(rB0, base + (ABLK + bb) * 512, bo);
      } else {
        const int bb = wid + 8 * (j - AJ);  // B block
        const int R = 8 * bb + (lane >> 3);
        const int kk = k0 + ((lane & 7) ^ swz(R)) * 8;
        const bool up = GATEUP && (j - AJ) * 64 >= kBN / 2;  // rows >= 128
        const int br = up ? bsrc(R) - kBN / 2 : bsrc(R);
        uint32_t bo = kk < K ? (uint32_t)(boff + br) * rowbytes + kk * (uint32_t)sizeof(S) : OOB;
        // an opaque copy of the offset: without it the compiler turned the
        // K-tail select into a branch around the last B loads, which cut
        // the region the scheduling groups order (forward 1-2 % faster)
        asm volatile("" : "+v"(bo));
        buffer_load_lds16(up ? rB1 : rB0, base + (ABLK + bb) * 512, bo);
      }
    }
  };

  // ---- fragments, MFMAs and the epilogue ---------------------------------------
  // The B tile row (LDS row) feeding column j of a lane's MFMA tiles is
  // brow0 + bstep(j), and all of them share one chunk rotation, so every
  // B fragment read is one base address plus a constant.
  // Plain products: column j of a lane is output column (lane % 16) * 8 + j
  // of the wave's 128, so after the K loop each lane holds 8 consecutive
  // outputs of a row and the epilogue stores them as one 16-byte vector.
  // Gate+up: column j < 4 is gate column (lane % 16) * 4 + j of the wave's
  // 64 act columns and j >= 4 the up column of the same act column, so each
  // lane holds 4 consecutive act outputs of a row.
  // (Plain products: B row wn * 128 + (lane % 16) * 8 + j sits at LDS row
  // wn * 128 + 64 * ((lane / 8) % 2) + 8 j + lane % 8; gate+up: gate row
  // wn * 64 + (lane % 16) * 4 + j at LDS row wn * 64 + 16 j + lane % 16.)
  const int brow0 = GATEUP ? wn * (TN / 2) + (lane & 15)
                           : wn * TN + ((lane >> 3) & 1) * 64 + (lane & 7);
  auto bstep = [](int j) -> int {
    constexpr int H2 = FN / 2;
    return GATEUP ? (j < H2 ? 16 * j : kBN / 2 + 16 * (j - H2)) : 8 * j;
  };
  const int bswz = swz(brow0);

  const int nk = (K + kBK - 1) / kBK;
  // Weight gradients: the fragment of columns c0 .. c0+15 (c0 a multiple
  // of 16) of a K-major stage part, at K rows 32 half +
  // 8 (lane / 16) + 0..7, from two transposing 8-byte LDS reads.  In each
  // 16-lane group, source lane s addresses K row 4 rd + s / 4 of the
  // group's 8 and columns c0 + 4 (s % 4) .. + 3, so the 16 lanes read 128
  // contiguous bytes (one slot of four rows: no bank conflict); lane
  // 4 r + p receives column c0 + 4 r + p of those four rows.
  auto tr_frag = [&](const S* T, int half, int c0) -> V {
    typedef short s4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s4 lds_s4;
    s4 t[2];
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int kq = 8 * half + 2 * (lane >> 4) + rd;  // group of 4 K rows
      const S* p = T + kq * kWgGroup + (c0 >> 4) * 64 + 4 * (lane & 15);
      t[rd] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)p);
    }
    V v;
    __builtin_memcpy(&v, t, sizeof(v));
    return v;
  };
  // NN: the B fragment of columns c0 .. c0+15 (c0 = 128 wn + 16 j) at K
  // rows 32 half + 8 (lane / 16) + 0..7, from two transposing reads of the
  // K-major B part (slots rotated by (q / 2) % 2 = (lane / 16) % 2; the
  // rotation flips bit 0 of the slot, j's parity, so the address stays a
  // per-lane base plus a constant)
  auto tr_frag_nn = [&](const S* T, int half, int c0) -> V {
    typedef short s4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s4 lds_s4;
    const int xo = ((lane >> 4) & 1) * 64;
    s4 t[2];
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int kq = 8 * half + 2 * (lane >> 4) + rd;
      const S* p = T + kq * 4 * kBN + (c0 >> 4) * 64 +
                   (((c0 >> 4) & 1) ? -xo : xo) + 4 * (lane & 15);
      t[rd] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)p);
    }
    V v;
    __builtin_memcpy(&v, t, sizeof(v));
    return v;
  };
  // Weight gradients multiply with the operands swapped (B fragment as the
  // MFMA's first operand): the accumulators then hold the transposed tile,
  // so lane l has Cw row (l % 16) and 4 consecutive columns 4 (l / 16) + q.
  auto mm = [](V a, V b, f32x4 c) -> f32x4 {
    if constexpr (WG) return Frag<D>::mma(b, a, c);
    else return Frag<D>::mma(a, b, c);
  };
  // The K loop and epilogue of a wave with FMC MFMA row tiles (0: it only
  // loads).  Each count has its own accumulators, so a wave with fewer row
  // tiles holds no idle accumulator registers.
  auto kloop = [&](auto fm_c) {
    constexpr int FMC = decltype(fm_c)::value;
    constexpr int FA = FMC > 0 ? FMC : 1;
    f32x4 acc[FA][FN];
#pragma unroll
    for (int i = 0; i < FA; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto read_frags = [&](int st, int half, V* fa, V* fb) {
      const S* As = sm + st * kStage;
      const S* Bs = As + kBM * kBK;
      if constexpr (WG) {
#pragma unroll
        for (int i = 0; i < FMC; ++i)
          fa[i] = tr_frag(As, half, tr0 + 16 * i);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          fb[j] = tr_frag(As + kWgPart, half, wn * TN + 16 * j);
        return;
      }
      const int c = half * 4 + (lane >> 4);
#pragma unroll
      for (int i = 0; i < FMC; ++i) {
        const int r = tr0 + i * 16 + (lane & 15);
        fa[i] = *(const V*)&As[r * kBK + ((c ^ swz(r)) << 3)];
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (NN)
          fb[j] = tr_frag_nn(Bs, half, wn * TN + 16 * j);
        else
          fb[j] = *(const V*)&Bs[(brow0 + bstep(j)) * kBK + ((c ^ bswz) << 3)];
      }
    };
    auto mma = [&](const V* fa, const V* fb) {
#pragma unroll
      for (int i = 0; i < FMC; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mm(fa[i], fb[j], acc[i][j]);
    };
    dma(0, 0);
    if (nk > 1) {
      // both first stages in flight before the first wait, so stage 1's
      // latency overlaps stage 0's; a raw barrier, because __syncthreads'
      // release fence would wait for stage 1 as well
      dma(kBK, 1);
      // the count leaves one stage's loads in flight
      if constexpr (BLK == 9)
        asm volatile("s_waitcnt vmcnt(9)\n\ts_barrier" ::: "memory");
      else {
        static_assert(BLK == 8, "one stage's loads per wave");
        asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
      }
    } else {
      wait_vmem();
      __syncthreads();
    }
    if constexpr (FMC > 0 && FMC <= 4) {
      // The second half of stage kt is multiplied after the barrier, while
      // the first half of stage kt+1 is read from LDS into the other
      // register set, so the matrix pipe has work while those reads land
      // (1-2 % faster).  With 5 row tiles the second register set does not
      // fit in 256 VGPRs, so that count keeps the plain order below.
      // The last K step is peeled off: with it inside the loop, the branch
      // that skips the barrier joins the barrier path just before the
      // second-half MFMAs, and the wait counts merged at that join made
      // them wait for the next stage's fragment reads as well.
      // Scheduling groups interleave the loads with the MFMAs: one MFMA
      // between consecutive LDS fragment reads before the barrier, and
      // after it one MFMA between consecutive operand loads, then between
      // the fragment reads.  Without them the compiler issued every load
      // and read first and the matrix pipe idled while both waves of a
      // SIMD did so (Mixtral-shaped expert stage 5 % faster with them).
      // The operand loads are issued unconditionally (the stage past the
      // last one reads zeros into a buffer nothing reads), so the region
      // after the barrier is one basic block the groups can order.
      V fa0[FMC], fb0[FN], fa1[FMC], fb1[FN];
      read_frags(0, 0, fa0, fb0);
      for (int kt = 0; kt + 1 < nk; ++kt) {
        const int st = kt & 1;
        read_frags(st, 1, fa1, fb1);
        mma(fa0, fb0);
#pragma unroll
        for (int q = 0; q < FMC + FN; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, FMC * FN > FMC + FN ? FMC * FN - (FMC + FN) : 0, 0);
        wait_vmem();
        __syncthreads();  // stage kt+1 landed everywhere; stage kt fully read
        dma((kt + 2) * kBK, st);  // past the last stage: zeros, never read
        read_frags(st ^ 1, 0, fa0, fb0);
        mma(fa1, fb1);
#pragma unroll
        for (int q = 0; q < BLK; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 1);
        }
#pragma unroll
        for (int q = 0; q < FMC + FN; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, FMC * FN > BLK + FMC + FN ? FMC * FN - BLK - FMC - FN : 0, 1);
      }
      wait_vmem();  // the zero loads past the last stage
      read_frags((nk - 1) & 1, 1, fa1, fb1);
      mma(fa0, fb0);
      mma(fa1, fb1);
    } else if constexpr (FMC > 4) {
      // Five row tiles: a second fragment set does not fit beside the 160
      // accumulators in 256 VGPRs.  One set is reloaded in place for the
      // next half while the current one is multiplied: the MFMAs of a half
      // go column by column, each B fragment is reloaded right after its
      // column, and each A fragment right after its MFMAs of the last two
      // columns (taken row by row).
      // The barrier sits between the halves and the last K step is peeled,
      // as above.
      auto read_a = [&](int st, int half, int i) -> V {
        if constexpr (WG)
          return tr_frag(sm + st * kStage, half, tr0 + 16 * i);
        const S* As = sm + st * kStage;
        const int c = half * 4 + (lane >> 4);
        const int r = tr0 + i * 16 + (lane & 15);
        return *(const V*)&As[r * kBK + ((c ^ swz(r)) << 3)];
      };
      auto read_b = [&](int st, int half, int j) -> V {
        if constexpr (WG)
          return tr_frag(sm + st * kStage + kWgPart, half, wn * TN + 16 * j);
        if constexpr (NN)
          return tr_frag_nn(sm + st * kStage + kBM * kBK, half, wn * TN + 16 * j);
        const S* Bs = sm + st * kStage + kBM * kBK;
        const int c = half * 4 + (lane >> 4);
        return *(const V*)&Bs[(brow0 + bstep(j)) * kBK + ((c ^ bswz) << 3)];
      };
      V fa[FMC], fb[FN];
      auto mma_cols = [&](int st2, int half2, bool reload) {
#pragma unroll
        for (int j = 0; j < FN - 2; ++j) {
#pragma unroll
          for (int i = 0; i < FMC; ++i)
            acc[i][j] = mm(fa[i], fb[j], acc[i][j]);
          if (reload) fb[j] = read_b(st2, half2, j);
        }
        // the last two columns row by row, so each A fragment is reloaded
        // eight MFMAs before the next half needs it
#pragma unroll
        for (int i = 0; i < FMC; ++i) {
#pragma unroll
          for (int j = FN - 2; j < FN; ++j)
            acc[i][j] = mm(fa[i], fb[j], acc[i][j]);
          if (reload) fa[i] = read_a(st2, half2, i);
        }
        if (reload) {
          fb[FN - 2] = read_b(st2, half2, FN - 2);
          fb[FN - 1] = read_b(st2, half2, FN - 1);
        }
      };
#pragma unroll
      for (int i = 0; i < FMC; ++i) fa[i] = read_a(0, 0, i);
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[j] = read_b(0, 0, j);
      for (int kt = 0; kt + 1 < nk; ++kt) {
        const int st = kt & 1;
        mma_cols(st, 1, true);  // first half; fragments of the second
        wait_vmem();
        __syncthreads();  // stage kt+1 landed everywhere; stage kt fully read
        dma((kt + 2) * kBK, st);  // past the last stage: zeros, never read
        mma_cols(st ^ 1, 0, true);  // second half; fragments of the next
        // one MFMA between consecutive operand loads, as above
#pragma unroll
        for (int q = 0; q < BLK; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
      }
      wait_vmem();  // the zero loads past the last stage
      mma_cols((nk - 1) & 1, 1, true);
      mma_cols(0, 0, false);
    } else {
      for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & 1;
        if constexpr (FMC > 0) {
          V fa[FMC], fb[FN];
          read_frags(st, 0, fa, fb);
          mma(fa, fb);
          read_frags(st, 1, fa, fb);
          mma(fa, fb);
        }
        if (kt + 1 < nk) {
          wait_vmem();
          __syncthreads();  // stage kt+1 landed everywhere; stage kt fully read
          if (kt + 2 < nk) dma((kt + 2) * kBK, st);
        }
      }
    }

    if constexpr (WG) {
      // M arrives as the kernel's K argument; K is now the expert's rows
#pragma unroll
      for (int i = 0; i < FMC; ++i) {
        const int64_t r = row0 + tr0 + i * 16 + (lane & 15);
        if (r >= tend) continue;
        float* cw = Cw + ((int64_t)e * Mw + r) * NB;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int64_t c = n0 + wn * TN + 16 * j + 4 * (lane >> 4);
          if (c < NB) *(f32x4*)(cw + c) = acc[i][j];
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < FMC; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t r = row0 + tr0 + i * 16 + (lane >> 4) * 4 + q;
        if (r >= tend) continue;
        // NB is a multiple of 8: a lane's group of 8 (weight gradients: each
        // of its two groups of 4) consecutive columns is wholly inside or
        // wholly past NB
        S* crow = C + r * NB;
        if (GATEUP) {
          // act columns 4 (lane % 16) .. + 3 of the wave's 64: one 8-byte
          // store (they were 16 apart, four 2-byte stores: the epilogue
          // took 14 % of a Mixtral-shaped gate+up tile)
          constexpr int H2 = FN / 2;
          const int64_t c0 = n0 + wn * (TN / 2) + (lane & 15) * H2;
          if (c0 < NB) {
            S v[H2];
#pragma unroll
            for (int j = 0; j < H2; ++j) {
              const float g = to_f32<D>(from_f32<D>(acc[i][j][q]));
              const float u = to_f32<D>(from_f32<D>(acc[i][j + H2][q]));
              v[j] = from_f32<D>(swiglu_act_t<CLIP>(g, u, sw));
            }
            u32x2 pk;
            __builtin_memcpy(&pk, v, sizeof(pk));
            *(u32x2*)(crow + c0) = pk;
          }
        } else if constexpr (NN) {
          // column j of a lane is output column 16 j + lane % 16
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int64_t c = n0 + wn * TN + 16 * j + (lane & 15);
            if (c < NB) crow[c] = from_f32<D>(acc[i][j][q]);
          }
        } else {
          const int64_t c0 = n0 + wn * TN + (lane & 15) * FN;
          if (c0 < NB) {
            V v;
#pragma unroll
            for (int j = 0; j < FN; ++j) v[j] = from_f32<D>(acc[i][j][q]);
            *(V*)(crow + c0) = v;
          }
        }
      }
    }
  };
  static_assert(kFM == 5, "the cases below cover 0..kFM row tiles");
  switch (fm) {
    case 5: kloop(std::integral_constant<int, 5>{}); break;
    case 4: kloop(std::integral_constant<int, 4>{}); break;
    case 3: kloop(std::integral_constant<int, 3>{}); break;
    case 2: kloop(std::integral_constant<int, 2>{}); break;
    case 1: kloop(std::integral_constant<int, 1>{}); break;
    default: kloop(std::integral_constant<int, 0>{}); break;
  }
}

template <int D, bool GATEUP>
hipError_t launch_one(const void* A, const void* B0, const void* B1, void* C,
                      const uint32_t* offsets, int64_t N, int K, int NB,
                      int E, int nseg, hipStream_t st, Swiglu sw = Swiglu{},
                      Gather ga = Gather{}) {
  using S = typename Storage<D>::T;
  const uint32_t ncol = cdiv(NB, GATEUP ? kBN / 2 : kBN);
  const int split = GATEUP && ga.rows ? 0 : kSplitUnits;
  // sum over segments of the row blocks <= ceil(N / block) + nseg
  const uint32_t grid = tile_grid_chunked(
      ncol * (cdiv(N, split > 0 ? 256 : kBM) + (uint32_t)nseg));
  // one instantiation per (gathering, activation) pair
  auto go = [&](auto gather_c, auto clip_c) -> hipError_t {
    constexpr bool G = decltype(gather_c)::value, CL = decltype(clip_c)::value;
    static std::atomic<uint64_t> attr{0};
    hipError_t err = allow_lds(
        (const void*)gemm_big_kernel<D, GATEUP, false, G, CL>, attr);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((gemm_big_kernel<D, GATEUP, false, G, CL>), dim3(grid),
                       dim3(512), kLds, st, (const S*)A, (const S*)B0,
                       (const S*)B1, (S*)C, offsets, N, K, NB, E, ncol, nseg,
                       nullptr, sw, G ? ga : Gather{}, split);
    return hipGetLastError();
  };
  using T = std::true_type;
  using F = std::false_type;
  if constexpr (GATEUP) {
    const bool clip = sw.limit >= 0.0f;
    if (ga.rows) return clip ? go(T{}, T{}) : go(T{}, F{});
    return clip ? go(F{}, T{}) : go(F{}, F{});
  } else {
    return go(F{}, F{});
  }
}

template <int D>
hipError_t launch_pair(const void* xd, int64_t N, int64_t H, int64_t I,
                       int E, const void* wg, const void* wu, const void* wd,
                       const uint32_t* offsets, void* act, void* y,
                       hipStream_t st, Swiglu sw, Gather ga) {
  hipError_t err = launch_one<D, true>(xd, wg, wu, act, offsets, N, (int)H,
                                       (int)I, E, E, st, sw, ga);
  if (err != hipSuccess) return err;
  timing_mark(5, st);
  return launch_one<D, false>(act, wd, wd, y, offsets, N, (int)I, (int)H, E,
                              E + 1, st);
}

}  // namespace

hipError_t launch_wgrad_big(const void* A, int dt, int64_t N, int M,
                            const void* B, int NC, int E,
                            const uint32_t* offsets, float* Cw,
                            hipStream_t st) {
  const uint32_t ncol = cdiv(NC, kBN);
  const uint32_t nmb = cdiv(M, kWgBM);
  const uint32_t grid = tile_grid_chunked((uint32_t)E * nmb * ncol, kWgChunk);
  if (dt == DT_BF16) {
    using S = typename Storage<DT_BF16>::T;
    static std::atomic<uint64_t> attr{0};
    hipError_t err =
        allow_lds((const void*)gemm_big_kernel<DT_BF16, false, true>, attr);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((gemm_big_kernel<DT_BF16, false, true>), dim3(grid),
                       dim3(512), kLds, st, (const S*)A, (const S*)B,
                       (const S*)B, (S*)nullptr, offsets, N, M, NC, E, ncol, 0,
                       Cw);
  } else {
    using S = typename Storage<DT_F16>::T;
    static std::atomic<uint64_t> attr{0};
    hipError_t err =
        allow_lds((const void*)gemm_big_kernel<DT_F16, false, true>, attr);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((gemm_big_kernel<DT_F16, false, true>), dim3(grid),
                       dim3(512), kLds, st, (const S*)A, (const S*)B,
                       (const S*)B, (S*)nullptr, offsets, N, M, NC, E, ncol, 0,
                       Cw);
  }
  return hipGetLastError();
}

hipError_t launch_nt_big(const void* A, int dt, int64_t N, int K,
                         const void* B, int NB, int E,
                         const uint32_t* offsets, void* C, hipStream_t st) {
  // segment E covers the rows past offsets[E]: they are written as zeros
  if (dt == DT_BF16)
    return launch_one<DT_BF16, false>(A, B, B, C, offsets, N, K, NB, E, E + 1,
                                      st);
  return launch_one<DT_F16, false>(A, B, B, C, offsets, N, K, NB, E, E + 1,
                                   st);
}

// C = A . B_e per segment with B stored K-major ([E, K, NB]): the NN form.
hipError_t launch_nn_big(const void* A, int dt, int64_t N, int K,
                         const void* B, int NB, int E,
                         const uint32_t* offsets, void* C, hipStream_t st) {
  const uint32_t ncol = cdiv(NB, kBN);
  const int nseg = E + 1;  // rows past offsets[E] are written as zeros
  const uint32_t grid =
      tile_grid_chunked(ncol * (cdiv(N, 256) + (uint32_t)nseg));
  auto go = [&](auto d_c) -> hipError_t {
    constexpr int DD = decltype(d_c)::value;
    using S = typename Storage<DD>::T;
    static std::atomic<uint64_t> attr{0};
    hipError_t err = allow_lds(
        (const void*)gemm_big_kernel<DD, false, false, false, true>, attr);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((gemm_big_kernel<DD, false, false, false, true>),
                       dim3(grid), dim3(512), kLds, st, (const S*)A,
                       (const S*)B, (const S*)B, (S*)C, offsets, N, K, NB, E,
                       ncol, nseg, nullptr, Swiglu{}, Gather{}, kSplitUnits);
    return hipGetLastError();
  };
  if (dt == DT_BF16) return go(std::integral_constant<int, DT_BF16>{});
  return go(std::integral_constant<int, DT_F16>{});
}

hipError_t launch_experts_big(const void* xd, int dt, int64_t N, int64_t H,
                              int64_t I, int E, const void* w_gate,
                              const void* w_up, const void* w_down,
                              const uint32_t* offsets, void* act, void* y,
                              hipStream_t st, Swiglu sw, Gather ga) {
  if (dt == DT_BF16)
    return launch_pair<DT_BF16>(xd, N, H, I, E, w_gate, w_up, w_down, offsets,
                                act, y, st, sw, ga);
  return launch_pair<DT_F16>(xd, N, H, I, E, w_gate, w_up, w_down, offsets,
                             act, y, st, sw, ga);
}

}  // namespace moe
