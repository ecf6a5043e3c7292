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

hipError_t launch_dispatch(const void* x, int dt, int64_t T, int64_t H,
                           int E, int k, const uint32_t* idx, void* xd,
                           uint32_t* offsets, uint32_t* row_expert,
                           uint32_t* row_token, uint32_t* token_row,
                           void* workspace, const DispatchPlan& plan,
                           hipStream_t st);

// ---- experts ---------------------------------------------------------------
hipError_t launch_experts(const void* xd, int dt, int64_t N, int64_t H,
                          int64_t I, int E, const void* w_gate,
                          const void* w_up, const void* w_down,
                          const uint32_t* offsets, void* act, void* y,
                          hipStream_t st);

// 256x256-tile kernels for prefill-sized segments (bf16/f16, H and I
// multiples of 8, 16-byte aligned, every per-expert weight matrix and 256
// rows of either operand under 2 GB).
hipError_t launch_experts_big(const void* xd, int dt, int64_t N, int64_t H,
                              int64_t I, int E, const void* w_gate,
                              const void* w_up, const void* w_down,
                              const uint32_t* offsets, void* act, void* y,
                              hipStream_t st);

// ---- combine ---------------------------------------------------------------
hipError_t launch_combine(const void* y, int dt, int64_t N, int64_t T,
                          int64_t H, int k, const void* w, int wdt,
                          const uint32_t* token_row, void* out,
                          hipStream_t st);

}  // namespace moe
