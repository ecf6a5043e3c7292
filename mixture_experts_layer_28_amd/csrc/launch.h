// Internal launchers of the libmoe kernels.  Host code only calls these after
// every argument has been validated; each returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---- instrumentation -------------------------------------------------------
// Records the n-th timing mark on `st` if the caller installed events
// (moe_set_timing_events); a no-op otherwise.
void timing_mark(int n, hipStream_t st);

// ---- routing ---------------------------------------------------------------
hipError_t launch_route(const void* logits, int ldt, int64_t T, int E, int k,
                        int renorm, uint32_t* idx, void* w, hipStream_t st);

// Options of group-limited sigmoid routing, validated by the caller:
// groups * gsz == E, 1 <= selected <= groups, gsz >= 2 if top_two.
struct GroupRouting {
  int groups;    // number of expert groups
  int gsz;       // experts per group
  int selected;  // groups kept per row
  int top_two;   // group score: sum of the two largest (else the largest)
  int renorm;    // renormalise the chosen weights
  float scale;   // applied after renormalisation
};
// E <= 1024, k <= 64; bias may be null.
hipError_t launch_route_sigmoid(const void* logits, int ldt, const float* bias,
                                int64_t T, int E, int k,
                                const GroupRouting& o, uint32_t* idx, void* w,
                                hipStream_t st);

// Router weights of a fixed selection and their logits gradient.  Index
// element types (values as in moe.h's moe_index_type):
enum IndexType { IDX_U32 = 0, IDX_I32 = 1, IDX_I64 = 2 };
// 1 <= k <= min(E, 64); sigmoid selects the scoring (else softmax).
hipError_t launch_selected_router_weights(const void* logits, int ldt,
                                          int64_t T, int E, const void* ind,
                                          int it, int k, int sigmoid,
                                          int renorm, float scale, float* w,
                                          hipStream_t st);
hipError_t launch_selected_router_backward(const void* logits, int ldt,
                                           int64_t T, int E, const void* ind,
                                           int it, int k, const float* grad_w,
                                           int sigmoid, int renorm,
                                           float scale, void* grad_x,
                                           hipStream_t st);

// ---- dispatch --------------------------------------------------------------
// Scratch layout: a table of per-chunk expert counts [nchunks][E+1] u32,
// reused in place for the per-chunk row bases.
struct DispatchPlan {
  int64_t N;        // T * k entries
  int64_t chunk;    // entries per chunk (multiple of 64)
  int64_t nchunks;  // ceil(N / chunk)
  int waves;        // chunks (waves) per count workgroup
  size_t table_bytes;
};
DispatchPlan plan_dispatch(int64_t T, int64_t E, int64_t k);

// xd == nullptr: the mapping only, no row copies (the expert GEMM then
// reads the token rows in place through row_token).
hipError_t launch_dispatch(const void* x, int dt, int64_t T, int64_t H,
                           int E, int k, const uint32_t* idx, void* xd,
                           uint32_t* offsets, uint32_t* row_expert,
                           uint32_t* row_token, uint32_t* token_row,
                           void* workspace, const DispatchPlan& plan,
                           hipStream_t st, bool counted = false);
// Softmax routing and the count step of `plan` in one launch (then
// launch_dispatch with counted = true): where k divides the plan's chunk,
// E <= kMaxFusedE and a chunk's ids and counters fit kMaxFusedLds u32 of
// LDS.  Writes idx, w, the count table and the per-chunk ranks exactly as
// launch_route followed by the count kernel does.
constexpr int kMaxFusedE = 1024;
constexpr int64_t kMaxFusedLds = 8192;
bool route_count_fusable(int E, int k, const DispatchPlan& plan);
hipError_t launch_route_count(const void* logits, int ldt, int64_t T, int E,
                              int k, int renorm, uint32_t* idx, void* w,
                              const DispatchPlan& plan, uint32_t* table,
                              uint32_t* local_rank, hipStream_t st);
// The static count table of moe_dispatch_noalloc: its size, and its device
// address on the current device (looked up once per device, never
// allocated).
size_t dispatch_scratch_bytes();
hipError_t dispatch_scratch(void** ptr);

// ---- experts ---------------------------------------------------------------
// Activation of the gate+up epilogue: limit < 0 is the plain SiLU(g) * u;
// otherwise the clipped form, gate clamped from above at limit, up to
// [-limit, limit], swish with parameter alpha of the clamped gate.
struct Swiglu {
  float alpha = 1.0f;
  float limit = -1.0f;
};

// Rows of the gate+up product's A operand read in place from the token
// rows: dispatched row r of the segments is row rows[r] of x [xrows, H]
// (the dispatch's row_token), so the dispatched copy xd is never
// materialised.  rows == nullptr: A is xd itself.
struct Gather {
  const uint32_t* rows = nullptr;
  int64_t xrows = 0;
};

hipError_t launch_experts(const void* xd, int dt, int64_t N, int64_t H,
                          int64_t I, int E, const void* w_gate,
                          const void* w_up, const void* w_down,
                          const uint32_t* offsets, void* act, void* y,
                          hipStream_t st, Swiglu sw = Swiglu{},
                          Gather ga = Gather{});
// Whether launch_experts takes its A rows through a Gather for these sizes
// and pointers (the MFMA paths, with x [xrows, H] addressable by 32-bit
// byte offsets, and for prefill-sized segments at most kGatherMaxColBlocks
// gate+up column blocks); otherwise xd is materialised.
bool experts_can_gather(int dt, int64_t N, int64_t H, int64_t I, int E,
                        int64_t xrows, const void* x, const void* w_gate,
                        const void* w_up, const void* w_down, const void* act,
                        const void* y);

// 256x256-tile kernels for prefill-sized segments (bf16/f16, H and I
// multiples of 8, 16-byte aligned, every per-expert weight matrix and 256
// rows of either operand under 2 GB).
hipError_t launch_experts_big(const void* xd, int dt, int64_t N, int64_t H,
                              int64_t I, int E, const void* w_gate,
                              const void* w_up, const void* w_down,
                              const uint32_t* offsets, void* act, void* y,
                              hipStream_t st, Swiglu sw = Swiglu{},
                              Gather ga = Gather{});

// One plain grouped NT product C[r, :] = A[r, :] . B[e]^T for the rows r of
// segment e (A [N,K], B [E,NB,K], C [N,NB], all of dtype dt); rows past
// offsets[E] are written as zeros.  Picks the same kernels as
// launch_experts.
hipError_t launch_grouped_nt(const void* A, int dt, int64_t N, int64_t K,
                             const void* B, int64_t NB, int E,
                             const uint32_t* offsets, void* C, hipStream_t st);
// The prefill-sized kernel of launch_experts_big for a plain product (bf16
// or f16; the same size limits).
hipError_t launch_nt_big(const void* A, int dt, int64_t N, int K,
                         const void* B, int NB, int E,
                         const uint32_t* offsets, void* C, hipStream_t st);
// ... its NN form: C = A . B_e with B stored K-major ([E, K, NB]), read
// through the LDS's transposing reads; the same types and limits.
hipError_t launch_nn_big(const void* A, int dt, int64_t N, int K,
                         const void* B, int NB, int E,
                         const uint32_t* offsets, void* C, hipStream_t st);

// ---- training path ---------------------------------------------------------
// Training forward: gate, up [N,I] (the raw products), act [N,I], y [N,H].
hipError_t launch_experts_forward_training(
    const void* xd, int dt, int64_t N, int64_t H, int64_t I, int E,
    const void* w_gate, const void* w_up, const void* w_down,
    const uint32_t* offsets, void* gate, void* up, void* act, void* y,
    hipStream_t st);
// Combine backward: dexp [N,H] (dtype dt), dw [T,k] FP32.
hipError_t launch_combine_backward(const void* y, int dt, int64_t N,
                                   int64_t T, int64_t H, int k,
                                   const void* w, int wdt,
                                   const uint32_t* token_row,
                                   const void* dout, void* dexp, float* dw,
                                   hipStream_t st);
// Expert backward scratch: one transposed weight tensor, then dact, dg, du
// [N,I], the two input-gradient halves [N,H], and two per-expert transposed
// operand copies of N * max(H, I) elements (byte offsets, 256-aligned).
struct ExpertsBackwardLayout {
  size_t wt, dact, dg, du, dxg, dxu, total;
};
ExpertsBackwardLayout experts_backward_layout(int64_t N, int64_t H,
                                              int64_t I, int64_t E, int dt);
hipError_t launch_experts_backward(
    const void* xd, int dt, int64_t N, int64_t H, int64_t I, int E,
    const void* w_gate, const void* w_up, const void* w_down,
    const uint32_t* offsets, const void* gate, const void* up,
    const void* act, const void* dy, void* dxd, float* dwg, float* dwu,
    float* dwd, void* workspace, hipStream_t st);

// Weight gradients on MFMA: Cw[e] [M, NC] FP32 = A_e^T . B_e where A_e and
// B_e are the rows [lo, lo + n_e) of expert e of A [N, M] and B [N, NC],
// read in place (K-major, K = n_e).  bf16/f16; M, NC multiples of 8;
// 16-byte aligned; N * max(M, NC) * 2 < 2^31.
hipError_t launch_wgrad_big(const void* A, int dt, int64_t N, int M,
                            const void* B, int NC, int E,
                            const uint32_t* offsets, float* Cw,
                            hipStream_t st);

// ---- combine ---------------------------------------------------------------
hipError_t launch_combine(const void* y, int dt, int64_t N, int64_t T,
                          int64_t H, int k, const void* w, int wdt,
                          const uint32_t* token_row, void* out,
                          hipStream_t st);

}  // namespace moe
