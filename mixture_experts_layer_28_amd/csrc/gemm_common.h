// Device helpers shared by the grouped-GEMM kernels (gemm.hip,
// gemm_big.hip): the device-side tile map, the LDS swizzle, the MFMA
// fragment types and the SwiGLU epilogue.
#pragma once

#include "device_common.h"
#include "launch.h"


namespace moe {

struct TileInfo {
  int64_t lo, hi, row0;  // segment [lo, hi); the tile's first row
  int e, col, found;
  int rows;              // rows of the tile: [row0, row0 + rows)
};

// Segment s < E is [offsets[s], offsets[s+1]); segment E (only if
// nseg > E) is [offsets[E], N).  Bounds are clamped into [0, N] and made
// monotone so that any offsets array keeps every access in bounds.
__device__ __forceinline__ void segment(const uint32_t* __restrict__ offsets,
                                        int s, int E, int64_t N, int nseg,
                                        int64_t* lo, int64_t* hi) {
  *lo = *hi = 0;
  if (s < nseg) {
    int64_t a = offsets[s];
    a = a < N ? a : N;
    int64_t b = s < E ? (int64_t)offsets[s + 1] : N;
    b = b < a ? a : (b > N ? N : b);
    *lo = a;
    *hi = b;
  }
}

// Consecutive logical tiles per XCD chunk (locate_tile).  Chunks of 8 and
// 32, groups of 2, 4 or 16 row blocks and the segments of fewer than 64 or
// 320 rows placed last measured the same or slower.
constexpr uint32_t kXcdChunk = 16;

__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// Tile map, executed by the 64 lanes of wavefront 0 of workgroup b of G.
//
// The tiles are (segment, row block, column block); only the segment sizes
// on the device fix how many exist, so the grid is an upper bound.  A
// segment of R rows has ceil(R / BM) row blocks: of BM rows each (the last
// one shorter) or, with `balanced`, made of the ceil(R / 32) units of 32
// rows (the last unit partial) dealt out as evenly as possible, so that no
// row block is a thin remainder (BM a multiple of 32).  The logical tiles
// are dealt to the 8 XCDs (hardware deals workgroup b to XCD b % 8) in
// chunks of kXcdChunk consecutive logical tiles, round robin: the tiles of
// one chunk run side by side on one XCD and share its L2, and every XCD
// gets a mix of large and small tiles.  (Contiguous ranges of equal tile
// counts per XCD left the XCD holding the most large tiles of a skewed
// routing ~9 % above the mean; the fine-grained expert stage ran 7 %
// faster with chunks of 16.)  One pass over the segments (a wave prefix
// sum of their tile counts) finds the segment of workgroup b's logical
// tile L.  Inside a segment, tiles go in groups of up to 8 row
// blocks: all column blocks of a group before the next group, the row
// blocks of one column block consecutive.
// G must be at least tile_grid(tiles).  BM is a template argument so that
// the per-segment block counts divide by a constant (a 64-bit division by
// a runtime value is a long instruction sequence).
//
// With `split` > 0 (balanced blocks only), a segment whose ceil(R / BM)
// blocks would average more than `split` units is cut into ceil(units / 8)
// blocks instead, of at most 8 units (256 rows): then G must be at least
// tile_grid_chunked over ceil(N / 256) + segments row blocks.
__device__ __forceinline__ uint32_t row_blocks(uint32_t R32, uint32_t nt,
                                               int split) {
  const uint32_t u = R32 / 32u + (R32 % 32u != 0);  // no wrap near 2^32
  return split > 0 && u > (uint32_t)split * nt ? (u + 7u) / 8u : nt;
}

template <int BM>
__device__ inline void locate_tile(uint32_t b, uint32_t G,
                                   const uint32_t* __restrict__ offsets,
                                   int E, int64_t N, uint32_t ncol,
                                   int nseg, TileInfo* ti,
                                   bool balanced = false, int split = 0) {
  const int lane = threadIdx.x;
  if (lane == 0) ti->found = 0;
  // the deal does not depend on the total: one pass over the segments
  // finds logical tile L, and an L past the last tile finds none
  const uint32_t local = b / 8u, q = local / kXcdChunk;
  const uint32_t L = (q * 8u + b % 8u) * kXcdChunk + local % kXcdChunk;
  (void)G;
  uint32_t base = 0;
  for (int s0 = 0; s0 < nseg; s0 += 64) {
    const int s = s0 + lane;
    int64_t lo, hi;
    segment(offsets, s, E, N, nseg, &lo, &hi);
    const uint32_t R32 = (uint32_t)(hi - lo);  // N < 2^32
    const uint32_t nt =
        row_blocks(R32, R32 / BM + (R32 % BM != 0), balanced ? split : 0);
    const uint32_t cnt = nt * ncol;
    const uint32_t inc = wave_inclusive_sum(cnt, lane);
    const uint32_t exc = inc - cnt;
    const bool hit = L >= base + exc && L < base + inc;
    if (__ballot(hit)) {
      if (hit) {
        const uint32_t l = L - base - exc;
        constexpr uint32_t GM = 8;
        const uint32_t grp = l / (GM * ncol), first = grp * GM;
        const uint32_t gs = nt - first < GM ? nt - first : GM;
        const uint32_t rem = l - grp * GM * ncol;
        ti->e = s;
        ti->lo = lo;
        ti->hi = hi;
        ti->col = (int)(rem / gs);
        const int64_t rb = first + rem % gs, R = hi - lo;
        if (balanced) {
          // whole 32-row units dealt out evenly (the last unit may be
          // partial): a block's busiest SIMD carries ceil(rows / 32) of its
          // 16-row MFMA tiles, so whole units leave no slot idle
          const int64_t u = (R + 31) / 32;
          const int64_t a = 32 * (rb * u / nt);
          int64_t z = 32 * ((rb + 1) * u / nt);
          z = z < R ? z : R;
          ti->row0 = lo + a;
          ti->rows = (int)(z - a);
        } else {
          ti->row0 = lo + rb * BM;
          ti->rows = (int)(hi - ti->row0 < BM ? hi - ti->row0 : BM);
        }
        ti->found = 1;
      }
      return;
    }
    base += __shfl(inc, 63, 64);
  }
}

// Grid for an upper bound of `tiles` tiles: a multiple of 8 with at least
// ceil(tiles / 8) workgroups on every XCD (the per-wave tile map of the
// decode kernels, which keeps contiguous XCD ranges).
inline uint32_t tile_grid(uint32_t tiles) { return 8u * ((tiles + 7u) / 8u); }
// ... for a chunked deal (locate_tile's: chunk = kXcdChunk): every XCD
// holds up to ceil(chunks / 8) chunks of `chunk` tiles.
inline uint32_t tile_grid_chunked(uint32_t tiles,
                                  uint32_t chunk = kXcdChunk) {
  const uint32_t nch = (tiles + chunk - 1) / chunk;
  return 8u * chunk * ((nch + 7u) / 8u);
}

__device__ __forceinline__ int swz(int r) { return r & 7; }

template <int D> struct Frag;
template <> struct Frag<DT_BF16> {
  using V = bf16x8;
  static __device__ __forceinline__ f32x4 mma(V a, V b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Frag<DT_F16> {
  using V = f16x8;
  static __device__ __forceinline__ f32x4 mma(V a, V b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

// SiLU(g) * u = g / (1 + e^-g) * u with the hardware exp2 and reciprocal
// (v_exp_f32, v_rcp_f32: about 1 ulp each, 5 instructions).  The library
// expf and IEEE divide took about 30, and unrolled over a gate+up tile's
// epilogue they doubled the kernel's code (115 KB, past the instruction
// cache); results differ from them by a few float ulps, far below the
// bf16/f16 rounding that follows.  Limits behave alike: g -> -inf gives
// 0 * g (NaN at -inf itself, as g / inf), g -> +inf gives g.
__device__ __forceinline__ float sigmoid_fast(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.4426950408889634f));
}
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * sigmoid_fast(g) * u;
}

// The gate+up epilogue's activation (Swiglu in launch.h).  The clamps keep
// a NaN a NaN (a comparison with NaN is false).
__device__ __forceinline__ float swiglu_clipped(float g, float u, Swiglu sw) {
  const float L = sw.limit;
  const float gc = g > L ? L : g;
  const float uc = u < -L ? -L : (u > L ? L : u);
  return gc * sigmoid_fast(sw.alpha * gc) * uc;
}
__device__ __forceinline__ float swiglu_act(float g, float u, Swiglu sw) {
  return sw.limit < 0.0f ? silu_mul(g, u) : swiglu_clipped(g, u, sw);
}
// ... chosen at compile time: with the choice at run time the compiler
// evaluates both forms for every output and selects, which made the
// plain epilogue carry the clamps and the alpha product.
template <bool CLIP>
__device__ __forceinline__ float swiglu_act_t(float g, float u, Swiglu sw) {
  if constexpr (CLIP) return swiglu_clipped(g, u, sw);
  else return silu_mul(g, u);
}


inline uint32_t cdiv(int64_t a, int64_t b) { return (uint32_t)((a + b - 1) / b); }

// Raw buffer resource over [base, base + bytes): loads at offsets at or
// beyond `bytes` return zeros (the hardware range check), which the GEMMs
// use for K tails and for rows past a segment or a weight matrix.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base,
                                                          uint64_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFF0ull ? 0xFFFFFFF0u : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)n, 0x00020000);
}

// 16 bytes per lane from a buffer straight into LDS: lane i writes
// lds + 16*i (gfx950 buffer_load_dwordx4 ... lds).  The LDS address space
// cast exists on the device side only.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r,
                                                  void* lds, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
#endif
}

__device__ __forceinline__ void wait_vmem() {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#endif
}

}  // namespace moe
