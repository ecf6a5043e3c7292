// Kernels of the first-order MoE training path.
//
// Contract: ruDNN user guide (RUDA docs, German edition), section 12
// "first-order MoE training" (combine backward -> expert backward ->
// dispatch backward -> router backward), and the experts page (docs.rs
// "ruDNN 0.1.25 source, src/moe/experts.rs": forward_dispatched_training,
// ExpertTrainingCache::backward_with_strategy), which fixes what the
// training forward keeps (raw gate and up products, the activation) and the
// expert backward's order: the down projection's backward, a SwiGLU
// backward, the gate and up projections' backwards, and the sum of their
// input gradients.  Every tensor that order materialises is rounded to the
// storage dtype; weight gradients are FP32.
//
// The products run on the forward's grouped GEMMs:
//   gate = xd . Wg^T, up = xd . Wu^T            (training forward, NT)
//   dact = dy . Wd,  dxg = dg . Wg,  dxu = du . Wu
// The input gradients take the prefill kernel's NN form, which reads the
// weights K-major in place through the LDS's transposing reads; shapes it
// does not take (fp32, unaligned, decode-sized segments) go through a
// transposed weight copy (one read and one write of the weight tensor) and
// the NT kernels.  The weight gradients are
// "TN" products over each expert's rows,
//   ddown[e] = dy_e^T . act_e,  dgate[e] = dg_e^T . xd_e,  dup[e] = du_e^T . xd_e;
// with bf16/f16 the prefill GEMM kernel's weight-gradient form (gemm_big.hip)
// reads both operands in place, K-major (K is the expert's row count),
// through the LDS's transposing reads; fp32 and unaligned shapes use an
// LDS-tiled FP32 kernel (tn_kernel).  Elementwise
// kernels do the SwiGLU forward and backward and the final add.

#include <initializer_list>

#include "device_common.h"
#include "gemm_common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int64_t kMaxGrid = 1 << 20;  // grid-stride loops beyond this

inline unsigned capped(int64_t blocks) {
  return (unsigned)(blocks < kMaxGrid ? (blocks > 0 ? blocks : 1) : kMaxGrid);
}

// ---- transpose: out[e][c][r] = in[e][r][c] ---------------------------------
template <typename W>
__global__ __launch_bounds__(256) void transpose_kernel(
    const W* __restrict__ in, W* __restrict__ out, int64_t E, int64_t R,
    int64_t C) {
  __shared__ W tile[64][65];
  const int64_t nr = (R + 63) / 64, nc = (C + 63) / 64;
  const int64_t total = E * nr * nc;
  const int tx = threadIdx.x % 64, ty = threadIdx.x / 64;
  for (int64_t b = blockIdx.x; b < total; b += gridDim.x) {
    const int64_t e = b / (nr * nc);
    const int64_t rb = (b / nc) % nr, cb = b % nc;
    const W* src = in + e * R * C;
    W* dst = out + e * R * C;
    for (int i = ty; i < 64; i += 4) {
      const int64_t r = rb * 64 + i, c = cb * 64 + tx;
      if (r < R && c < C) tile[i][tx] = src[r * C + c];
    }
    __syncthreads();
    for (int i = ty; i < 64; i += 4) {
      const int64_t c = cb * 64 + i, r = rb * 64 + tx;
      if (r < R && c < C) dst[c * R + r] = tile[tx][i];
    }
    __syncthreads();
  }
}

// LDS tile of 64 x 64 16-bit elements for the 16-byte transposes: the
// 8-element vector v of row i sits in slot v ^ (i / 8 % 8), so that the
// column gathers below (8 lanes on 8 row groups of one column block) hit
// 32 different banks.
__device__ __forceinline__ int tslot(int i, int v) { return v ^ ((i >> 3) & 7); }
__device__ __forceinline__ uint16_t tread(const uint16_t (*tile)[64], int i,
                                          int j) {
  return tile[i][tslot(i, j >> 3) * 8 + (j & 7)];
}

// 16-bit elements, R and C multiples of 8, 16-byte aligned: 16-byte loads
// of 8 consecutive columns into the LDS tile, then 16-byte stores of 8
// consecutive rows of one column gathered from the tile; 8 neighbouring
// lanes store the 8 row groups of one column, one 128-byte line.
__global__ __launch_bounds__(256) void transpose16_kernel(
    const uint16_t* __restrict__ in, uint16_t* __restrict__ out, int64_t E,
    int64_t R, int64_t C) {
  __shared__ uint16_t tile[64][64];
  const int64_t nr = (R + 63) / 64, nc = (C + 63) / 64;
  const int64_t total = E * nr * nc;
  for (int64_t b = blockIdx.x; b < total; b += gridDim.x) {
    const int64_t e = b / (nr * nc);
    const int64_t r0 = ((b / nc) % nr) * 64, c0 = (b % nc) * 64;
    const uint16_t* src = in + e * R * C;
    uint16_t* dst = out + e * R * C;
    // 64 rows x 8 vectors: thread t loads rows t/8 and t/8 + 32, vector t%8
    for (int q = threadIdx.x; q < 512; q += 256) {
      const int i = q / 8, v = q % 8;
      const int64_t r = r0 + i, c = c0 + v * 8;
      if (r < R && c < C)
        *(u32x4*)&tile[i][tslot(i, v) * 8] = *(const u32x4*)(src + r * C + c);
    }
    __syncthreads();
    // 64 columns x 8 vectors of rows: column j, rows 8w .. 8w+7
    for (int q = threadIdx.x; q < 512; q += 256) {
      const int j = q / 8, w = q % 8;
      const int64_t c = c0 + j, r = r0 + w * 8;
      if (c < C && r < R) {
        uint16_t v[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) v[t] = tread(tile, w * 8 + t, j);
        *(u32x4*)(dst + c * R + r) = *(const u32x4*)v;
      }
    }
    __syncthreads();
  }
}

// ---- elementwise -----------------------------------------------------------
// NV consecutive elements per thread and step: 16-byte vectors when the
// caller checked that every array is 16-byte aligned and n % NV == 0,
// else NV = 1.
template <int D, int NV>
struct Chunk {
  using S = typename Storage<D>::T;
  S v[NV];
  __device__ __forceinline__ void load(const S* p) {
    if constexpr (NV * sizeof(S) == 16) *(u32x4*)v = *(const u32x4*)p;
    else
#pragma unroll
      for (int i = 0; i < NV; ++i) v[i] = p[i];
  }
  __device__ __forceinline__ void store(S* p) const {
    if constexpr (NV * sizeof(S) == 16) *(u32x4*)p = *(const u32x4*)v;
    else
#pragma unroll
      for (int i = 0; i < NV; ++i) p[i] = v[i];
  }
};

// act = SiLU(g) * u from the stored (rounded) g and u, as the forward's
// fused epilogue computes it.
template <int D, int NV>
__global__ __launch_bounds__(256) void swiglu_fwd_kernel(
    const typename Storage<D>::T* __restrict__ g,
    const typename Storage<D>::T* __restrict__ u,
    typename Storage<D>::T* __restrict__ a, int64_t n) {
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * NV; i < n;
       i += (int64_t)gridDim.x * 256 * NV) {
    Chunk<D, NV> cg, cu, ca;
    cg.load(g + i);
    cu.load(u + i);
#pragma unroll
    for (int q = 0; q < NV; ++q)
      ca.v[q] = from_f32<D>(silu_mul(to_f32<D>(cg.v[q]), to_f32<D>(cu.v[q])));
    ca.store(a + i);
  }
}

// SwiGLU backward of a = SiLU(g) * u, s = sigmoid(g):
//   dg = da * u * s * (1 + g * (1 - s)),  du = da * g * s
template <int D, int NV>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(
    const typename Storage<D>::T* __restrict__ g,
    const typename Storage<D>::T* __restrict__ u,
    const typename Storage<D>::T* __restrict__ da,
    typename Storage<D>::T* __restrict__ dg,
    typename Storage<D>::T* __restrict__ du, int64_t n) {
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * NV; i < n;
       i += (int64_t)gridDim.x * 256 * NV) {
    Chunk<D, NV> cg, cu, cd, og, ou;
    cg.load(g + i);
    cu.load(u + i);
    cd.load(da + i);
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const float gv = to_f32<D>(cg.v[q]), uv = to_f32<D>(cu.v[q]);
      const float d = to_f32<D>(cd.v[q]);
      const float s = 1.0f / (1.0f + expf(-gv));
      og.v[q] = from_f32<D>(d * uv * s * (1.0f + gv * (1.0f - s)));
      ou.v[q] = from_f32<D>(d * gv * s);
    }
    og.store(dg + i);
    ou.store(du + i);
  }
}

template <int D, int NV>
__global__ __launch_bounds__(256) void add_kernel(
    const typename Storage<D>::T* __restrict__ a,
    const typename Storage<D>::T* __restrict__ b,
    typename Storage<D>::T* __restrict__ c, int64_t n) {
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * NV; i < n;
       i += (int64_t)gridDim.x * 256 * NV) {
    Chunk<D, NV> ca, cb, cc;
    ca.load(a + i);
    cb.load(b + i);
#pragma unroll
    for (int q = 0; q < NV; ++q)
      cc.v[q] = from_f32<D>(to_f32<D>(ca.v[q]) + to_f32<D>(cb.v[q]));
    cc.store(c + i);
  }
}

// ---- combine backward ------------------------------------------------------
// One workgroup (4 waves) per token; wave v takes slots v, v + 4, ...  For
// slot j with row r = token_row[t, j]: dexpert[r] = w[t, j] * dout[t]
// (rounded to the dtype) and dweights[t, j] = dout[t] . y[r] in FP32.  A
// row id >= N is not touched and gets a NaN weight gradient.  NV elements
// per load (16-byte vectors when the rows allow, else 1).
template <int D, int WD, int NV>
__global__ __launch_bounds__(256) void combine_bwd_kernel(
    const typename Storage<D>::T* __restrict__ y, int64_t N, int64_t T,
    int64_t H, int k, const typename Storage<WD>::T* __restrict__ w,
    const uint32_t* __restrict__ token_row,
    const typename Storage<D>::T* __restrict__ dout,
    typename Storage<D>::T* __restrict__ dexp, float* __restrict__ dw) {
  using S = typename Storage<D>::T;
  const int lane = threadIdx.x % 64, wv = threadIdx.x / 64;
  const int64_t vpr = H / NV;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    const S* go = dout + t * H;
    for (int j = wv; j < k; j += 4) {
      const uint32_t r = token_row[t * k + j];
      const float wt = to_f32<WD>(w[t * k + j]);
      float dot = 0.0f;
      if (r < (uint64_t)N) {
        const S* yr = y + (int64_t)r * H;
        S* dr = dexp + (int64_t)r * H;
        for (int64_t v = lane; v < vpr; v += 64) {
          S a[NV], b[NV], o[NV];
          if constexpr (NV * sizeof(S) == 16) {
            *(u32x4*)a = *(const u32x4*)(go + v * NV);
            *(u32x4*)b = *(const u32x4*)(yr + v * NV);
          } else {
#pragma unroll
            for (int i = 0; i < NV; ++i) {
              a[i] = go[v * NV + i];
              b[i] = yr[v * NV + i];
            }
          }
#pragma unroll
          for (int i = 0; i < NV; ++i) {
            const float gv = to_f32<D>(a[i]);
            dot = fmaf(gv, to_f32<D>(b[i]), dot);
            o[i] = from_f32<D>(wt * gv);
          }
          if constexpr (NV * sizeof(S) == 16) {
            *(u32x4*)(dr + v * NV) = *(const u32x4*)o;
          } else {
#pragma unroll
            for (int i = 0; i < NV; ++i) dr[v * NV + i] = o[i];
          }
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) dot += __shfl_xor(dot, o, 64);
      if (lane == 0) dw[t * k + j] = r < (uint64_t)N ? dot : __builtin_nanf("");
    }
  }
}

// ---- weight gradients: C[e] = A_e^T . B_e over the rows of segment e -------
// A [N,M], B [N,NC] (dtype), C [E,M,NC] FP32.  64 x 64 output tile per
// workgroup, 4 x 4 per thread, K (rows) in steps of 16 staged in LDS as
// FP32.  An empty segment writes zeros.
template <int D>
__global__ __launch_bounds__(256) void tn_kernel(
    const typename Storage<D>::T* __restrict__ A,
    const typename Storage<D>::T* __restrict__ B,
    const uint32_t* __restrict__ offsets, int64_t N, int E, int64_t M,
    int64_t NC, float* __restrict__ C) {
  constexpr int BK = 16;
  __shared__ float As[BK][64 + 4];
  __shared__ float Bs[BK][64 + 4];
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  const int64_t nm = (M + 63) / 64, nn = (NC + 63) / 64;
  const int64_t total = (int64_t)E * nm * nn;
  for (int64_t b = blockIdx.x; b < total; b += gridDim.x) {
    const int e = (int)(b / (nm * nn));
    const int64_t m0 = ((b / nn) % nm) * 64, c0 = (b % nn) * 64;
    int64_t hi = offsets[e + 1];
    hi = hi < N ? hi : N;
    int64_t lo = offsets[e];
    lo = lo < hi ? lo : hi;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
    for (int64_t r0 = lo; r0 < hi; r0 += BK) {
      // 16 rows x 64 columns of each operand, 4 per thread
      const int lr = threadIdx.x / 16, lc = (threadIdx.x % 16) * 4;
      const int64_t r = r0 + lr;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t m = m0 + lc + q, c = c0 + lc + q;
        As[lr][lc + q] = r < hi && m < M ? to_f32<D>(A[r * M + m]) : 0.0f;
        Bs[lr][lc + q] = r < hi && c < NC ? to_f32<D>(B[r * NC + c]) : 0.0f;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < BK; ++kk) {
        float a[4], bb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
        for (int j = 0; j < 4; ++j) bb[j] = Bs[kk][tx * 4 + j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], bb[j], acc[i][j]);
      }
      __syncthreads();
    }
    float* ce = C + (int64_t)e * M * NC;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0 + ty * 4 + i;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t c = c0 + tx * 4 + j;
        if (c < NC) ce[m * NC + c] = acc[i][j];
      }
    }
  }
}

template <typename W>
hipError_t transpose(const void* in, void* out, int64_t E, int64_t R,
                     int64_t C, hipStream_t st) {
  const int64_t blocks = E * ((R + 63) / 64) * ((C + 63) / 64);
  hipLaunchKernelGGL((transpose_kernel<W>), dim3(capped(blocks)), dim3(256), 0,
                     st, (const W*)in, (W*)out, E, R, C);
  return hipGetLastError();
}

hipError_t transpose_dt(const void* in, int dt, void* out, int64_t E,
                        int64_t R, int64_t C, hipStream_t st) {
  if (dt == DT_F32) return transpose<uint32_t>(in, out, E, R, C, st);
  if (R % 8 == 0 && C % 8 == 0 && ((uintptr_t)in | (uintptr_t)out) % 16 == 0) {
    const int64_t blocks = E * ((R + 63) / 64) * ((C + 63) / 64);
    hipLaunchKernelGGL(transpose16_kernel, dim3(capped(blocks)), dim3(256), 0,
                       st, (const uint16_t*)in, (uint16_t*)out, E, R, C);
    return hipGetLastError();
  }
  return transpose<uint16_t>(in, out, E, R, C, st);
}

template <int D>
hipError_t tn(const void* A, const void* B, const uint32_t* offsets,
              int64_t N, int E, int64_t M, int64_t NC, float* C,
              hipStream_t st) {
  using S = typename Storage<D>::T;
  const int64_t blocks = (int64_t)E * ((M + 63) / 64) * ((NC + 63) / 64);
  hipLaunchKernelGGL((tn_kernel<D>), dim3(capped(blocks)), dim3(256), 0, st,
                     (const S*)A, (const S*)B, offsets, N, E, M, NC, C);
  return hipGetLastError();
}

hipError_t tn_dt(const void* A, int dt, const void* B,
                 const uint32_t* offsets, int64_t N, int E, int64_t M,
                 int64_t NC, float* C, hipStream_t st) {
  switch (dt) {
    case DT_F32: return tn<DT_F32>(A, B, offsets, N, E, M, NC, C, st);
    case DT_F16: return tn<DT_F16>(A, B, offsets, N, E, M, NC, C, st);
    default: return tn<DT_BF16>(A, B, offsets, N, E, M, NC, C, st);
  }
}

// Weight gradient Cw[e] = A_e^T . B_e over each expert's rows (A [N,M],
// B [N,NC] in dtype dt): on MFMA, reading both operands K-major in place,
// when the shapes allow, else the FMA kernel.
hipError_t wgrad(const void* A, int dt, const void* B,
                 const uint32_t* offsets, int64_t N, int E, int64_t M,
                 int64_t NC, float* Cw, hipStream_t st) {
  const uintptr_t al = (uintptr_t)A | (uintptr_t)B | (uintptr_t)Cw;
  const bool mfma = dt != DT_F32 && M % 8 == 0 && NC % 8 == 0 &&
                    al % 16 == 0 &&
                    N * (M > NC ? M : NC) * 2 < ((int64_t)1 << 31);
  if (!mfma) return tn_dt(A, dt, B, offsets, N, E, M, NC, Cw, st);
  return launch_wgrad_big(A, dt, N, (int)M, B, (int)NC, E, offsets, Cw, st);
}

// 16-byte vectors when every pointer is 16-byte aligned and n is a whole
// number of vectors.
template <int D>
bool vec_ok(int64_t n, std::initializer_list<const void*> ps) {
  constexpr int NV = 16 / sizeof(typename Storage<D>::T);
  uintptr_t al = 0;
  for (const void* p : ps) al |= (uintptr_t)p;
  return n % NV == 0 && al % 16 == 0;
}

template <int D>
hipError_t elementwise_fwd(const void* g, const void* u, void* a, int64_t n,
                           hipStream_t st) {
  using S = typename Storage<D>::T;
  constexpr int NV = 16 / sizeof(S);
  if (vec_ok<D>(n, {g, u, a}))
    hipLaunchKernelGGL((swiglu_fwd_kernel<D, NV>),
                       dim3(capped((n / NV + 255) / 256)), dim3(256), 0, st,
                       (const S*)g, (const S*)u, (S*)a, n);
  else
    hipLaunchKernelGGL((swiglu_fwd_kernel<D, 1>),
                       dim3(capped((n + 255) / 256)), dim3(256), 0, st,
                       (const S*)g, (const S*)u, (S*)a, n);
  return hipGetLastError();
}

template <int D>
hipError_t elementwise_bwd(const void* g, const void* u, const void* da,
                           void* dg, void* du, int64_t n, hipStream_t st) {
  using S = typename Storage<D>::T;
  constexpr int NV = 16 / sizeof(S);
  if (vec_ok<D>(n, {g, u, da, dg, du}))
    hipLaunchKernelGGL((swiglu_bwd_kernel<D, NV>),
                       dim3(capped((n / NV + 255) / 256)), dim3(256), 0, st,
                       (const S*)g, (const S*)u, (const S*)da, (S*)dg,
                       (S*)du, n);
  else
    hipLaunchKernelGGL((swiglu_bwd_kernel<D, 1>),
                       dim3(capped((n + 255) / 256)), dim3(256), 0, st,
                       (const S*)g, (const S*)u, (const S*)da, (S*)dg,
                       (S*)du, n);
  return hipGetLastError();
}

template <int D>
hipError_t elementwise_add(const void* a, const void* b, void* c, int64_t n,
                           hipStream_t st) {
  using S = typename Storage<D>::T;
  constexpr int NV = 16 / sizeof(S);
  if (vec_ok<D>(n, {a, b, c}))
    hipLaunchKernelGGL((add_kernel<D, NV>),
                       dim3(capped((n / NV + 255) / 256)), dim3(256), 0, st,
                       (const S*)a, (const S*)b, (S*)c, n);
  else
    hipLaunchKernelGGL((add_kernel<D, 1>), dim3(capped((n + 255) / 256)),
                       dim3(256), 0, st, (const S*)a, (const S*)b, (S*)c, n);
  return hipGetLastError();
}

#define MOE_BY_DT(dt, fn, ...)                                     \
  ((dt) == DT_F32 ? fn<DT_F32>(__VA_ARGS__)                        \
                  : (dt) == DT_F16 ? fn<DT_F16>(__VA_ARGS__)       \
                                   : fn<DT_BF16>(__VA_ARGS__))

template <int D, int WD>
hipError_t combine_bwd(const void* y, int64_t N, int64_t T, int64_t H, int k,
                       const void* w, const uint32_t* token_row,
                       const void* dout, void* dexp, float* dw,
                       hipStream_t st) {
  using S = typename Storage<D>::T;
  using SW = typename Storage<WD>::T;
  constexpr int NV = 16 / sizeof(S);
  const uintptr_t al = (uintptr_t)y | (uintptr_t)dout | (uintptr_t)dexp;
  const dim3 grid(capped(T));
  if (H % NV == 0 && al % 16 == 0)
    hipLaunchKernelGGL((combine_bwd_kernel<D, WD, NV>), grid, dim3(256), 0, st,
                       (const S*)y, N, T, H, k, (const SW*)w, token_row,
                       (const S*)dout, (S*)dexp, dw);
  else
    hipLaunchKernelGGL((combine_bwd_kernel<D, WD, 1>), grid, dim3(256), 0, st,
                       (const S*)y, N, T, H, k, (const SW*)w, token_row,
                       (const S*)dout, (S*)dexp, dw);
  return hipGetLastError();
}

template <int D>
hipError_t combine_bwd_w(const void* y, int64_t N, int64_t T, int64_t H,
                         int k, const void* w, int wdt,
                         const uint32_t* token_row, const void* dout,
                         void* dexp, float* dw, hipStream_t st) {
  switch (wdt) {
    case DT_F32: return combine_bwd<D, DT_F32>(y, N, T, H, k, w, token_row, dout, dexp, dw, st);
    case DT_F16: return combine_bwd<D, DT_F16>(y, N, T, H, k, w, token_row, dout, dexp, dw, st);
    default: return combine_bwd<D, DT_BF16>(y, N, T, H, k, w, token_row, dout, dexp, dw, st);
  }
}

}  // namespace

hipError_t launch_experts_forward_training(
    const void* xd, int dt, int64_t N, int64_t H, int64_t I, int E,
    const void* w_gate, const void* w_up, const void* w_down,
    const uint32_t* offsets, void* gate, void* up, void* act, void* y,
    hipStream_t st) {
  hipError_t err = launch_grouped_nt(xd, dt, N, H, w_gate, I, E, offsets,
                                     gate, st);
  if (err == hipSuccess)
    err = launch_grouped_nt(xd, dt, N, H, w_up, I, E, offsets, up, st);
  if (err == hipSuccess)
    err = MOE_BY_DT(dt, elementwise_fwd, gate, up, act, N * I, st);
  if (err == hipSuccess)
    err = launch_grouped_nt(act, dt, N, I, w_down, H, E, offsets, y, st);
  return err;
}

hipError_t launch_combine_backward(const void* y, int dt, int64_t N,
                                   int64_t T, int64_t H, int k,
                                   const void* w, int wdt,
                                   const uint32_t* token_row,
                                   const void* dout, void* dexp, float* dw,
                                   hipStream_t st) {
  switch (dt) {
    case DT_F32: return combine_bwd_w<DT_F32>(y, N, T, H, k, w, wdt, token_row, dout, dexp, dw, st);
    case DT_F16: return combine_bwd_w<DT_F16>(y, N, T, H, k, w, wdt, token_row, dout, dexp, dw, st);
    default: return combine_bwd_w<DT_BF16>(y, N, T, H, k, w, wdt, token_row, dout, dexp, dw, st);
  }
}

ExpertsBackwardLayout experts_backward_layout(int64_t N, int64_t H,
                                              int64_t I, int64_t E, int dt) {
  const size_t s = dt == DT_F32 ? 4 : 2;
  ExpertsBackwardLayout L;
  size_t at = 0;
  auto take = [&](size_t bytes) {
    const size_t here = at;
    at = (at + bytes + 255) & ~size_t(255);
    return here;
  };
  L.wt = take((size_t)E * H * I * s);
  L.dact = take((size_t)N * I * s);
  L.dg = take((size_t)N * I * s);
  L.du = take((size_t)N * I * s);
  L.dxg = take((size_t)N * H * s);
  L.dxu = take((size_t)N * H * s);
  L.total = at;
  return L;
}

// C = A . W_e per segment, W [E, K, NB]: on the prefill kernel's NN form
// (W read K-major in place) when the shapes allow, else through a
// transposed copy of W in wt and the NT products.
hipError_t grouped_nn(const void* A, int dt, int64_t N, int64_t K,
                      const void* W, int64_t NB, int E,
                      const uint32_t* offsets, void* C, void* wt,
                      hipStream_t st) {
  const uintptr_t al = (uintptr_t)A | (uintptr_t)W | (uintptr_t)C;
  const int64_t lim = (int64_t)1 << 31;
  if (dt != DT_F32 && K % 8 == 0 && NB % 8 == 0 && al % 16 == 0 &&
      N >= 96 * (int64_t)E && K * NB * 2 < lim && 320 * K * 2 < lim)
    return launch_nn_big(A, dt, N, (int)K, W, (int)NB, E, offsets, C, st);
  hipError_t err = transpose_dt(W, dt, wt, E, K, NB, st);
  if (err == hipSuccess)
    err = launch_grouped_nt(A, dt, N, K, wt, NB, E, offsets, C, st);
  return err;
}

hipError_t launch_experts_backward(
    const void* xd, int dt, int64_t N, int64_t H, int64_t I, int E,
    const void* w_gate, const void* w_up, const void* w_down,
    const uint32_t* offsets, const void* gate, const void* up,
    const void* act, const void* dy, void* dxd, float* dwg, float* dwu,
    float* dwd, void* workspace, hipStream_t st) {
  const ExpertsBackwardLayout L = experts_backward_layout(N, H, I, E, dt);
  char* ws = (char*)workspace;
  void* wt = ws + L.wt;
  void* dact = ws + L.dact;
  void* dg = ws + L.dg;
  void* du = ws + L.du;
  void* dxg = ws + L.dxg;
  void* dxu = ws + L.dxu;
  // down projection: input gradient through Wd [E,H,I] read K-major (or a
  // transposed copy), weight gradient
  hipError_t err = grouped_nn(dy, dt, N, H, w_down, I, E, offsets, dact, wt,
                              st);
  if (err == hipSuccess)
    err = wgrad(dy, dt, act, offsets, N, E, H, I, dwd, st);
  // SwiGLU backward
  if (err == hipSuccess)
    err = MOE_BY_DT(dt, elementwise_bwd, gate, up, dact, dg, du, N * I, st);
  // gate and up projections: input gradients through Wg^T, Wu^T [E,H,I]
  // (one transposed copy at a time), weight gradients, then the sum
  if (err == hipSuccess)
    err = grouped_nn(dg, dt, N, I, w_gate, H, E, offsets, dxg, wt, st);
  if (err == hipSuccess)
    err = grouped_nn(du, dt, N, I, w_up, H, E, offsets, dxu, wt, st);
  if (err == hipSuccess)
    err = MOE_BY_DT(dt, elementwise_add, dxg, dxu, dxd, N * H, st);
  if (err == hipSuccess)
    err = wgrad(dg, dt, xd, offsets, N, E, I, H, dwg, st);
  if (err == hipSuccess)
    err = wgrad(du, dt, xd, offsets, N, E, I, H, dwu, st);
  return err;
}

}  // namespace moe
