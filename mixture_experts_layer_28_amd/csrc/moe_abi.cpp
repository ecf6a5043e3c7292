// C ABI of libmoe: argument checks, workspace arithmetic and launch order.
//
// Every check below runs on the host before anything is enqueued and never
// reads device memory.  The API mirrors the staged and one-call forms of the
// ruDNN MoE interface (ruDNN user guide, section 6 "calling MoE"; experts page
// SwiGluExperts::new / forward_dispatched_with_strategy / forward), whose
// MoeError results become status codes here.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/moe.h"
#include "launch.h"

namespace {

thread_local char g_last_error[512] = "";
thread_local hipEvent_t g_marks[MOE_TIMING_EVENTS];
thread_local int g_nmarks = 0;
thread_local bool g_in_forward = false;

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return MOE_OK;
}

int hip_status(hipError_t err, const char* what) {
  if (err == hipSuccess) return ok();
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

bool valid_dtype(int d) { return d == MOE_F32 || d == MOE_F16 || d == MOE_BF16; }
int64_t dsize(int d) { return d == MOE_F32 ? 4 : 2; }

// a * b without int64 overflow (both >= 0)
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}
bool bytes_ok(int64_t a, int64_t b, int64_t s) {
  int64_t t;
  return mul_ok(a, b, &t) && mul_ok(t, s, &t);
}

constexpr int64_t kMaxRows = 0xffffffffLL;  // row ids are uint32
constexpr int64_t kMaxRouteE = 65536;
constexpr int64_t kMaxDispatchE = 16383;    // count table fits LDS
constexpr int64_t kMaxCombineK = 8192;      // one token's row ids and weights
                                            // fit 64 KB of LDS

size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

int check_route(const void* logits, int ldt, int64_t T, int64_t E,
                int64_t k, const void* idx, const void* w) {
  if (!valid_dtype(ldt)) return fail(MOE_ERR_DTYPE, "moe_route: unknown logits dtype %d", ldt);
  if (T < 0) return fail(MOE_ERR_SHAPE, "moe_route: T must be >= 0");
  if (E < 1) return fail(MOE_ERR_SHAPE, "moe_route: E must be >= 1");
  if (E > kMaxRouteE) return fail(MOE_ERR_UNSUPPORTED, "moe_route: E > %lld", (long long)kMaxRouteE);
  if (k < 1 || k > E) return fail(MOE_ERR_INVALID_ARG, "moe_route: top_k must satisfy 1 <= top_k <= E");
  int64_t n;
  if (!mul_ok(T, k, &n) || n > kMaxRows) return fail(MOE_ERR_SHAPE, "moe_route: T*top_k must be < 2^32");
  if (!bytes_ok(T, E, 4)) return fail(MOE_ERR_SHAPE, "moe_route: T*E overflows");
  if (T > 0 && (!logits || !idx || !w)) return fail(MOE_ERR_INVALID_ARG, "moe_route: null pointer");
  return MOE_OK;
}

// Limits of group-limited sigmoid routing (guide, section 10).
constexpr int64_t kMaxSigmoidE = 1024;
constexpr int64_t kMaxGroups = 128;
constexpr int64_t kMaxSigmoidK = 64;

int check_route_sigmoid(const void* logits, int ldt, int64_t T, int64_t E,
                        int64_t k, int64_t groups, int64_t sel, int top_two,
                        float scale, const void* idx, const void* w) {
  const char* f = "moe_route_sigmoid_grouped";
  if (!valid_dtype(ldt)) return fail(MOE_ERR_DTYPE, "%s: unknown logits dtype %d", f, ldt);
  if (T < 0) return fail(MOE_ERR_SHAPE, "%s: T must be >= 0", f);
  if (E < 1 || E > kMaxSigmoidE) return fail(MOE_ERR_INVALID_ARG, "%s: E must be in 1..=%lld", f, (long long)kMaxSigmoidE);
  if (groups < 1 || groups > kMaxGroups || E % groups != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: groups must be in 1..=%lld and divide E", f, (long long)kMaxGroups);
  if (sel < 1 || sel > groups) return fail(MOE_ERR_INVALID_ARG, "%s: selected_groups must be in 1..=groups", f);
  if (k < 1 || k > kMaxSigmoidK || k > sel * (E / groups))
    return fail(MOE_ERR_INVALID_ARG, "%s: top_k must be in 1..=%lld and at most the experts of the selected groups", f, (long long)kMaxSigmoidK);
  if (top_two && E / groups < 2) return fail(MOE_ERR_INVALID_ARG, "%s: group_top_two needs two experts per group", f);
  if (!std::isfinite(scale) || !(scale > 0.0f)) return fail(MOE_ERR_INVALID_ARG, "%s: scale must be finite and positive", f);
  int64_t n;
  if (!mul_ok(T, k, &n) || n > kMaxRows) return fail(MOE_ERR_SHAPE, "%s: T*top_k must be < 2^32", f);
  if (!bytes_ok(T, E, 4)) return fail(MOE_ERR_SHAPE, "%s: T*E overflows", f);
  if (T > 0 && (!logits || !idx || !w)) return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", f);
  return MOE_OK;
}

int check_router_weights(const char* f, const void* logits, int ldt,
                         int64_t T, int64_t E, const void* ind, int it,
                         int64_t k, int scoring, float scale, const void* a,
                         const void* b) {
  if (!valid_dtype(ldt)) return fail(MOE_ERR_DTYPE, "%s: unknown logits dtype %d", f, ldt);
  if (it != MOE_IDX_U32 && it != MOE_IDX_I32 && it != MOE_IDX_I64)
    return fail(MOE_ERR_INVALID_ARG, "%s: unknown index type %d", f, it);
  if (scoring != MOE_SCORE_SOFTMAX && scoring != MOE_SCORE_SIGMOID)
    return fail(MOE_ERR_INVALID_ARG, "%s: unknown scoring %d", f, scoring);
  if (T < 0) return fail(MOE_ERR_SHAPE, "%s: T must be >= 0", f);
  if (E < 1 || E > INT32_MAX) return fail(MOE_ERR_INVALID_ARG, "%s: E must be in 1..2^31-1", f);
  if (k < 1 || k > E || k > kMaxSigmoidK)
    return fail(MOE_ERR_INVALID_ARG, "%s: top_k must satisfy 1 <= top_k <= min(E, 64)", f);
  if (!std::isfinite(scale) || !(scale > 0.0f)) return fail(MOE_ERR_INVALID_ARG, "%s: scale must be finite and positive", f);
  int64_t n;
  if (!mul_ok(T, k, &n) || !bytes_ok(T, k, 8) || !bytes_ok(T, E, 4))
    return fail(MOE_ERR_SHAPE, "%s: sizes overflow", f);
  if (T > 0 && (!logits || !ind || !a || !b)) return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", f);
  return MOE_OK;
}

moe::GroupRouting group_routing(int64_t E, int64_t groups, int64_t sel,
                                int top_two, int renorm, float scale) {
  moe::GroupRouting o;
  o.groups = (int)groups;
  o.gsz = (int)(E / groups);
  o.selected = (int)sel;
  o.top_two = top_two ? 1 : 0;
  o.renorm = renorm ? 1 : 0;
  o.scale = scale;
  return o;
}

int check_dispatch(const void* x, int dt, int64_t T, int64_t H, int64_t E,
                   int64_t k, const void* idx, const void* xd,
                   const void* offsets, const void* row_expert,
                   const void* row_token, const void* token_row) {
  if (!valid_dtype(dt)) return fail(MOE_ERR_DTYPE, "moe_dispatch: unknown dtype %d", dt);
  if (T < 0) return fail(MOE_ERR_SHAPE, "moe_dispatch: T must be >= 0");
  if (H < 1) return fail(MOE_ERR_SHAPE, "moe_dispatch: H must be >= 1");
  if (E < 1) return fail(MOE_ERR_SHAPE, "moe_dispatch: E must be >= 1");
  if (E > kMaxDispatchE) return fail(MOE_ERR_UNSUPPORTED, "moe_dispatch: E > %lld", (long long)kMaxDispatchE);
  if (k < 1 || k > E) return fail(MOE_ERR_INVALID_ARG, "moe_dispatch: top_k must satisfy 1 <= top_k <= E");
  int64_t n;
  if (!mul_ok(T, k, &n) || n > kMaxRows) return fail(MOE_ERR_SHAPE, "moe_dispatch: T*top_k must be < 2^32");
  if (!bytes_ok(n, H, dsize(dt))) return fail(MOE_ERR_SHAPE, "moe_dispatch: N*H overflows");
  if (!offsets) return fail(MOE_ERR_INVALID_ARG, "moe_dispatch: null offsets");
  if (T > 0 && (!x || !idx || !xd || !row_expert || !row_token || !token_row))
    return fail(MOE_ERR_INVALID_ARG, "moe_dispatch: null pointer");
  return MOE_OK;
}

int check_experts(const void* xd, int dt, int64_t N, int64_t H, int64_t I,
                  int64_t E, const void* wg, const void* wu, const void* wd,
                  const void* offsets, const void* act, const void* y) {
  if (!valid_dtype(dt)) return fail(MOE_ERR_DTYPE, "moe_experts_forward: unknown dtype %d", dt);
  if (N < 0) return fail(MOE_ERR_SHAPE, "moe_experts_forward: N must be >= 0");
  if (N > kMaxRows) return fail(MOE_ERR_SHAPE, "moe_experts_forward: N must be < 2^32");
  if (E < 1 || H < 1 || I < 1) return fail(MOE_ERR_SHAPE, "moe_experts_forward: E, H and I must be >= 1");
  if (H > INT32_MAX || I > INT32_MAX || E > kMaxDispatchE)
    return fail(MOE_ERR_UNSUPPORTED, "moe_experts_forward: H, I < 2^31 and E <= %lld required", (long long)kMaxDispatchE);
  int64_t ei;
  if (!mul_ok(E, I, &ei) || !bytes_ok(ei, H, dsize(dt)))
    return fail(MOE_ERR_SHAPE, "moe_experts_forward: weight size overflows");
  if (!bytes_ok(N, H > I ? H : I, dsize(dt))) return fail(MOE_ERR_SHAPE, "moe_experts_forward: N*max(H,I) overflows");
  if (!wg || !wu || !wd) return fail(MOE_ERR_INVALID_ARG, "moe_experts_forward: null weight pointer");
  if (N > 0 && (!xd || !act || !y || !offsets)) return fail(MOE_ERR_INVALID_ARG, "moe_experts_forward: null pointer");
  return MOE_OK;
}

int check_combine(const void* y, int dt, int64_t N, int64_t T, int64_t H,
                  int64_t k, const void* w, int wdt, const void* token_row,
                  const void* out) {
  if (!valid_dtype(dt) || !valid_dtype(wdt)) return fail(MOE_ERR_DTYPE, "moe_combine: unknown dtype");
  if (T < 0 || N < 0 || H < 1) return fail(MOE_ERR_SHAPE, "moe_combine: T, N >= 0 and H >= 1 required");
  if (k < 1) return fail(MOE_ERR_INVALID_ARG, "moe_combine: top_k must be >= 1");
  int64_t n;
  if (!mul_ok(T, k, &n) || n > kMaxRows || N > kMaxRows) return fail(MOE_ERR_SHAPE, "moe_combine: T*top_k and N must be < 2^32");
  if (!bytes_ok(N > T ? N : T, H, dsize(dt))) return fail(MOE_ERR_SHAPE, "moe_combine: size overflows");
  if (k > kMaxCombineK) return fail(MOE_ERR_UNSUPPORTED, "moe_combine: top_k > %lld", (long long)kMaxCombineK);
  if (T > 0 && (!y || !w || !token_row || !out)) return fail(MOE_ERR_INVALID_ARG, "moe_combine: null pointer");
  return MOE_OK;
}

struct ForwardLayout {
  size_t idx, w, offsets, row_expert, row_token, token_row, xd, dws, act, y,
      total;
};

ForwardLayout forward_layout(int64_t T, int64_t H, int64_t I, int64_t E,
                             int64_t k, int dt, int ldt) {
  ForwardLayout L;
  const int64_t N = T * k;
  size_t at = 0;
  auto take = [&](size_t bytes) {
    const size_t here = at;
    at = align_up(at + bytes);
    return here;
  };
  L.idx = take((size_t)N * 4);
  L.w = take((size_t)N * dsize(ldt));
  L.offsets = take((size_t)(E + 1) * 4);
  L.row_expert = take((size_t)N * 4);
  L.row_token = take((size_t)N * 4);
  L.token_row = take((size_t)N * 4);
  L.xd = take((size_t)N * H * dsize(dt));
  L.dws = take(moe::plan_dispatch(T, E, k).table_bytes);
  L.act = take((size_t)N * I * dsize(dt));
  L.y = take((size_t)N * H * dsize(dt));
  L.total = at;
  return L;
}

}  // namespace

namespace moe {
void timing_mark(int n, hipStream_t st) {
  if (g_in_forward && g_nmarks == MOE_TIMING_EVENTS && n >= 0 &&
      n < g_nmarks && g_marks[n])
    (void)hipEventRecord(g_marks[n], st);
}
}  // namespace moe

// The stages after routing, shared by the forwards: the checks that do
// not depend on the routing method, the workspace carve-up and the launch
// sequence.  `route(idx, w, stream, plan, table, rank, &counted)` launches
// the routing kernel; where it also ran the dispatch count of `plan` into
// table/rank (one launch instead of two) it sets counted.
template <typename Route>
int run_forward(const char* f, const void* x, int dt, int ldt, int64_t T,
                int64_t H, int64_t I, int64_t E, int64_t top_k,
                const void* w_gate, const void* w_up, const void* w_down,
                void* out, void* workspace, size_t workspace_bytes,
                void* stream, Route route, moe::Swiglu sw = moe::Swiglu{}) {
  // x stands in for the workspace-resident offsets/act/y buffers here;
  // the workspace itself is checked below.
  int s = check_experts(x, dt, T * top_k, H, I, E, w_gate, w_up, w_down, x, x, x);
  if (s != MOE_OK) return s;
  if (T > 0 && (!x || !out)) return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", f);
  if (top_k > kMaxCombineK) return fail(MOE_ERR_UNSUPPORTED, "%s: top_k > %lld", f, (long long)kMaxCombineK);
  const size_t need = moe_forward_workspace_size(T, H, I, E, top_k, dt, ldt);
  if (need == 0) return fail(MOE_ERR_SHAPE, "%s: sizes out of range", f);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_INVALID_ARG, "%s: workspace needs %zu bytes", f, need);
  if ((uintptr_t)workspace % 256 != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", f);
  if (T == 0) return ok();

  const ForwardLayout L = forward_layout(T, H, I, E, top_k, dt, ldt);
  char* ws = (char*)workspace;
  uint32_t* idx = (uint32_t*)(ws + L.idx);
  void* w = ws + L.w;
  uint32_t* offsets = (uint32_t*)(ws + L.offsets);
  uint32_t* row_expert = (uint32_t*)(ws + L.row_expert);
  uint32_t* row_token = (uint32_t*)(ws + L.row_token);
  uint32_t* token_row = (uint32_t*)(ws + L.token_row);
  void* xd = ws + L.xd;
  void* dws = ws + L.dws;
  void* act = ws + L.act;
  void* y = ws + L.y;
  const int64_t N = T * top_k;
  const hipStream_t st = (hipStream_t)stream;
  char what[96];

  struct Marking {
    Marking() { g_in_forward = true; }
    ~Marking() { g_in_forward = false; }
  } marking;
  const moe::DispatchPlan plan = moe::plan_dispatch(T, E, top_k);
  bool counted = false;
  moe::timing_mark(0, st);
  hipError_t err = route(idx, w, st, plan, (uint32_t*)dws, token_row, &counted);
  std::snprintf(what, sizeof(what), "%s(route)", f);
  if (err != hipSuccess) return hip_status(err, what);
  // Where the MFMA kernels can read the token rows in place, dispatch
  // writes only the mapping and the gate+up GEMM gathers its A rows from x
  // through row_token (the same values as the copies, so the same result).
  const bool gather = moe::experts_can_gather(dt, N, H, I, (int)E, T, x,
                                              w_gate, w_up, w_down, act, y);
  moe::timing_mark(1, st);
  err = moe::launch_dispatch(x, dt, T, H, (int)E, (int)top_k, idx,
                             gather ? nullptr : xd, offsets, row_expert,
                             row_token, token_row, dws, plan, st, counted);
  std::snprintf(what, sizeof(what), "%s(dispatch)", f);
  if (err != hipSuccess) return hip_status(err, what);
  moe::timing_mark(4, st);
  moe::Gather ga;
  if (gather) {
    ga.rows = row_token;
    ga.xrows = T;
  }
  err = moe::launch_experts(gather ? x : xd, dt, N, H, I, (int)E, w_gate,
                            w_up, w_down, offsets, act, y, st, sw, ga);
  std::snprintf(what, sizeof(what), "%s(experts)", f);
  if (err != hipSuccess) return hip_status(err, what);
  moe::timing_mark(6, st);
  err = moe::launch_combine(y, dt, N, T, H, (int)top_k, w, ldt, token_row,
                            out, st);
  moe::timing_mark(7, st);
  std::snprintf(what, sizeof(what), "%s(combine)", f);
  return hip_status(err, what);
}

extern "C" {

int moe_set_timing_events(void* const* events, int count) {
  if (count == 0) {
    g_nmarks = 0;
    return ok();
  }
  if (count != MOE_TIMING_EVENTS || !events)
    return fail(MOE_ERR_INVALID_ARG, "moe_set_timing_events: need %d events", MOE_TIMING_EVENTS);
  for (int i = 0; i < count; ++i) g_marks[i] = (hipEvent_t)events[i];  // NULL: mark skipped
  g_nmarks = count;
  return ok();
}


const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_SHAPE: return "invalid or overflowing shape";
    case MOE_ERR_DTYPE: return "unknown dtype";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_last_error; }

int moe_route(const void* logits, int ldt, int64_t T, int64_t E,
              int64_t top_k, int renormalize, uint32_t* idx, void* weights,
              void* stream) {
  const int s = check_route(logits, ldt, T, E, top_k, idx, weights);
  if (s != MOE_OK) return s;
  if (T == 0) return ok();
  return hip_status(moe::launch_route(logits, ldt, T, (int)E, (int)top_k,
                                      renormalize ? 1 : 0, idx, weights,
                                      (hipStream_t)stream),
                    "moe_route");
}

size_t moe_dispatch_workspace_size(int64_t T, int64_t E, int64_t top_k) {
  int64_t n;
  if (T < 0 || E < 1 || E > kMaxDispatchE || top_k < 1 || top_k > E ||
      !mul_ok(T, top_k, &n) || n > kMaxRows)
    return 0;
  return align_up(moe::plan_dispatch(T, E, top_k).table_bytes) + 256;
}

int moe_dispatch(const void* x, int dt, int64_t T, int64_t H, int64_t E,
                 int64_t top_k, const uint32_t* idx, void* xd,
                 uint32_t* offsets, uint32_t* row_expert, uint32_t* row_token,
                 uint32_t* token_row, void* workspace, size_t workspace_bytes,
                 void* stream) {
  int s = check_dispatch(x, dt, T, H, E, top_k, idx, xd, offsets, row_expert,
                         row_token, token_row);
  if (s != MOE_OK) return s;
  const size_t need = moe_dispatch_workspace_size(T, E, top_k);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_INVALID_ARG, "moe_dispatch: workspace needs %zu bytes", need);
  if ((uintptr_t)workspace % 4 != 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_dispatch: workspace must be 4-byte aligned");
  const moe::DispatchPlan plan = moe::plan_dispatch(T, E, top_k);
  // T == 0 still writes offsets (all zero): every segment is empty.
  return hip_status(
      moe::launch_dispatch(x, dt, T, H, (int)E, (int)top_k, idx, xd, offsets,
                           row_expert, row_token, token_row, workspace, plan,
                           (hipStream_t)stream),
      "moe_dispatch");
}

int moe_dispatch_noalloc(const void* x, int dt, int64_t T, int64_t H,
                         int64_t E, int64_t top_k, const uint32_t* idx,
                         void* xd, uint32_t* offsets, uint32_t* row_expert,
                         uint32_t* row_token, uint32_t* token_row,
                         void* stream) {
  int s = check_dispatch(x, dt, T, H, E, top_k, idx, xd, offsets, row_expert,
                         row_token, token_row);
  if (s != MOE_OK) return s;
  const moe::DispatchPlan plan = moe::plan_dispatch(T, E, top_k);
  const size_t cap = moe::dispatch_scratch_bytes();
  if (plan.table_bytes > cap)
    return fail(MOE_ERR_UNSUPPORTED,
                "moe_dispatch_noalloc: the count table needs %zu bytes, more "
                "than the %zu-byte static scratch (use moe_dispatch)",
                plan.table_bytes, cap);
  void* table = nullptr;
  hipError_t err = moe::dispatch_scratch(&table);
  if (err != hipSuccess) return hip_status(err, "moe_dispatch_noalloc");
  return hip_status(
      moe::launch_dispatch(x, dt, T, H, (int)E, (int)top_k, idx, xd, offsets,
                           row_expert, row_token, token_row, table, plan,
                           (hipStream_t)stream),
      "moe_dispatch_noalloc");
}

int moe_experts_forward(const void* xd, int dt, int64_t N, int64_t H,
                        int64_t I, int64_t E, const void* w_gate,
                        const void* w_up, const void* w_down,
                        const uint32_t* offsets, void* act, void* y,
                        void* stream) {
  const int s = check_experts(xd, dt, N, H, I, E, w_gate, w_up, w_down,
                              offsets, act, y);
  if (s != MOE_OK) return s;
  if (N == 0) return ok();
  return hip_status(moe::launch_experts(xd, dt, N, H, I, (int)E, w_gate, w_up,
                                        w_down, offsets, act, y,
                                        (hipStream_t)stream),
                    "moe_experts_forward");
}

int moe_experts_forward_clipped(const void* xd, int dt, int64_t N, int64_t H,
                                int64_t I, int64_t E, const void* w_gate,
                                const void* w_up, const void* w_down,
                                const uint32_t* offsets, float alpha,
                                float limit, void* act, void* y,
                                void* stream) {
  const int s = check_experts(xd, dt, N, H, I, E, w_gate, w_up, w_down,
                              offsets, act, y);
  if (s != MOE_OK) return s;
  if (!std::isfinite(alpha))
    return fail(MOE_ERR_INVALID_ARG, "moe_experts_forward_clipped: alpha must be finite");
  if (!std::isfinite(limit) || !(limit >= 0.0f))
    return fail(MOE_ERR_INVALID_ARG, "moe_experts_forward_clipped: limit must be finite and >= 0");
  if (N == 0) return ok();
  moe::Swiglu sw;
  sw.alpha = alpha;
  sw.limit = limit;
  return hip_status(moe::launch_experts(xd, dt, N, H, I, (int)E, w_gate, w_up,
                                        w_down, offsets, act, y,
                                        (hipStream_t)stream, sw),
                    "moe_experts_forward_clipped");
}

int moe_combine(const void* y, int dt, int64_t N, int64_t T, int64_t H,
                int64_t top_k, const void* weights, int wdt,
                const uint32_t* token_row, void* out, void* stream) {
  const int s = check_combine(y, dt, N, T, H, top_k, weights, wdt, token_row,
                              out);
  if (s != MOE_OK) return s;
  if (T == 0) return ok();
  return hip_status(moe::launch_combine(y, dt, N, T, H, (int)top_k, weights,
                                        wdt, token_row, out,
                                        (hipStream_t)stream),
                    "moe_combine");
}

size_t moe_forward_workspace_size(int64_t T, int64_t H, int64_t I, int64_t E,
                                  int64_t top_k, int dt, int ldt) {
  if (!valid_dtype(dt) || !valid_dtype(ldt) || T < 0 || H < 1 || I < 1 ||
      E < 1 || E > kMaxDispatchE || top_k < 1 || top_k > E)
    return 0;
  int64_t n;
  if (!mul_ok(T, top_k, &n) || n > kMaxRows ||
      !bytes_ok(n, H > I ? H : I, 16))
    return 0;
  return forward_layout(T, H, I, E, top_k, dt, ldt).total;
}

int moe_forward(const void* x, int dt, const void* logits, int ldt,
                int64_t T, int64_t H, int64_t I, int64_t E, int64_t top_k,
                int renormalize, const void* w_gate, const void* w_up,
                const void* w_down, void* out, void* workspace,
                size_t workspace_bytes, void* stream) {
  const int s = check_route(logits, ldt, T, E, top_k, workspace, workspace);
  if (s != MOE_OK) return s;
  return run_forward(
      "moe_forward", x, dt, ldt, T, H, I, E, top_k, w_gate, w_up, w_down, out,
      workspace, workspace_bytes, stream,
      [&](uint32_t* idx, void* w, hipStream_t st, const moe::DispatchPlan& p,
          uint32_t* table, uint32_t* rank, bool* counted) {
        if (moe::route_count_fusable((int)E, (int)top_k, p)) {
          *counted = true;
          return moe::launch_route_count(logits, ldt, T, (int)E, (int)top_k,
                                         renormalize ? 1 : 0, idx, w, p,
                                         table, rank, st);
        }
        return moe::launch_route(logits, ldt, T, (int)E, (int)top_k,
                                 renormalize ? 1 : 0, idx, w, st);
      });
}

int moe_forward_clipped(const void* x, int dt, const void* logits, int ldt,
                        int64_t T, int64_t H, int64_t I, int64_t E,
                        int64_t top_k, int renormalize, float alpha,
                        float limit, const void* w_gate, const void* w_up,
                        const void* w_down, void* out, void* workspace,
                        size_t workspace_bytes, void* stream) {
  const int s = check_route(logits, ldt, T, E, top_k, workspace, workspace);
  if (s != MOE_OK) return s;
  if (!std::isfinite(alpha))
    return fail(MOE_ERR_INVALID_ARG, "moe_forward_clipped: alpha must be finite");
  if (!std::isfinite(limit) || !(limit >= 0.0f))
    return fail(MOE_ERR_INVALID_ARG, "moe_forward_clipped: limit must be finite and >= 0");
  moe::Swiglu sw;
  sw.alpha = alpha;
  sw.limit = limit;
  return run_forward(
      "moe_forward_clipped", x, dt, ldt, T, H, I, E, top_k, w_gate, w_up,
      w_down, out, workspace, workspace_bytes, stream,
      [&](uint32_t* idx, void* w, hipStream_t st, const moe::DispatchPlan& p,
          uint32_t* table, uint32_t* rank, bool* counted) {
        if (moe::route_count_fusable((int)E, (int)top_k, p)) {
          *counted = true;
          return moe::launch_route_count(logits, ldt, T, (int)E, (int)top_k,
                                         renormalize ? 1 : 0, idx, w, p,
                                         table, rank, st);
        }
        return moe::launch_route(logits, ldt, T, (int)E, (int)top_k,
                                 renormalize ? 1 : 0, idx, w, st);
      },
      sw);
}

int moe_route_sigmoid_grouped(const void* logits, int ldt, int64_t T,
                              int64_t E, const float* bias, int64_t top_k,
                              int64_t groups, int64_t selected_groups,
                              int group_top_two, int renormalize, float scale,
                              uint32_t* idx, void* weights, void* stream) {
  const int s = check_route_sigmoid(logits, ldt, T, E, top_k, groups,
                                    selected_groups, group_top_two, scale,
                                    idx, weights);
  if (s != MOE_OK) return s;
  if (T == 0) return ok();
  const moe::GroupRouting o = group_routing(E, groups, selected_groups,
                                            group_top_two, renormalize, scale);
  return hip_status(moe::launch_route_sigmoid(logits, ldt, bias, T, (int)E,
                                              (int)top_k, o, idx, weights,
                                              (hipStream_t)stream),
                    "moe_route_sigmoid_grouped");
}

int moe_forward_sigmoid_grouped(const void* x, int dt, const void* logits,
                                int ldt, const float* bias, int64_t T,
                                int64_t H, int64_t I, int64_t E,
                                int64_t top_k, int64_t groups,
                                int64_t selected_groups, int group_top_two,
                                int renormalize, float scale,
                                const void* w_gate, const void* w_up,
                                const void* w_down, void* out,
                                void* workspace, size_t workspace_bytes,
                                void* stream) {
  const int s = check_route_sigmoid(logits, ldt, T, E, top_k, groups,
                                    selected_groups, group_top_two, scale,
                                    workspace, workspace);
  if (s != MOE_OK) return s;
  const moe::GroupRouting o = group_routing(E, groups, selected_groups,
                                            group_top_two, renormalize, scale);
  return run_forward(
      "moe_forward_sigmoid_grouped", x, dt, ldt, T, H, I, E, top_k, w_gate,
      w_up, w_down, out, workspace, workspace_bytes, stream,
      [&](uint32_t* idx, void* w, hipStream_t st, const moe::DispatchPlan&,
          uint32_t*, uint32_t*, bool*) {
        return moe::launch_route_sigmoid(logits, ldt, bias, T, (int)E,
                                         (int)top_k, o, idx, w, st);
      });
}

int moe_selected_router_weights(const void* logits, int ldt, int64_t T,
                                int64_t E, const void* indices,
                                int index_type, int64_t top_k, int scoring,
                                int renormalize, float scale, float* weights,
                                void* stream) {
  const int s = check_router_weights("moe_selected_router_weights", logits,
                                     ldt, T, E, indices, index_type, top_k,
                                     scoring, scale, weights, weights);
  if (s != MOE_OK) return s;
  if (T == 0) return ok();
  return hip_status(moe::launch_selected_router_weights(
                        logits, ldt, T, (int)E, indices, index_type,
                        (int)top_k, scoring == MOE_SCORE_SIGMOID,
                        renormalize ? 1 : 0, scale, weights,
                        (hipStream_t)stream),
                    "moe_selected_router_weights");
}

int moe_selected_router_backward(const void* logits, int ldt, int64_t T,
                                 int64_t E, const void* indices,
                                 int index_type, int64_t top_k,
                                 const float* grad_weights, int scoring,
                                 int renormalize, float scale,
                                 void* grad_logits, void* stream) {
  const int s = check_router_weights("moe_selected_router_backward", logits,
                                     ldt, T, E, indices, index_type, top_k,
                                     scoring, scale, grad_weights,
                                     grad_logits);
  if (s != MOE_OK) return s;
  if (T == 0) return ok();
  return hip_status(moe::launch_selected_router_backward(
                        logits, ldt, T, (int)E, indices, index_type,
                        (int)top_k, grad_weights,
                        scoring == MOE_SCORE_SIGMOID, renormalize ? 1 : 0,
                        scale, grad_logits, (hipStream_t)stream),
                    "moe_selected_router_backward");
}

int moe_experts_forward_training(const void* xd, int dt, int64_t N,
                                 int64_t H, int64_t I, int64_t E,
                                 const void* w_gate, const void* w_up,
                                 const void* w_down, const uint32_t* offsets,
                                 void* gate, void* up, void* act, void* y,
                                 void* stream) {
  const int s = check_experts(xd, dt, N, H, I, E, w_gate, w_up, w_down,
                              offsets, act, y);
  if (s != MOE_OK) return s;
  if (N > 0 && (!gate || !up))
    return fail(MOE_ERR_INVALID_ARG, "moe_experts_forward_training: null pointer");
  if (N == 0) return ok();
  return hip_status(moe::launch_experts_forward_training(
                        xd, dt, N, H, I, (int)E, w_gate, w_up, w_down,
                        offsets, gate, up, act, y, (hipStream_t)stream),
                    "moe_experts_forward_training");
}

int moe_combine_backward(const void* y, int dt, int64_t N, int64_t T,
                         int64_t H, int64_t top_k, const void* weights,
                         int wdt, const uint32_t* token_row,
                         const void* grad_out, void* grad_expert,
                         float* grad_weights, void* stream) {
  const int s = check_combine(y, dt, N, T, H, top_k, weights, wdt, token_row,
                              grad_out);
  if (s != MOE_OK) return s;
  if (T > 0 && (!grad_expert || !grad_weights))
    return fail(MOE_ERR_INVALID_ARG, "moe_combine_backward: null pointer");
  if (T == 0) return ok();
  return hip_status(moe::launch_combine_backward(
                        y, dt, N, T, H, (int)top_k, weights, wdt, token_row,
                        grad_out, grad_expert, grad_weights,
                        (hipStream_t)stream),
                    "moe_combine_backward");
}

size_t moe_experts_backward_workspace_size(int64_t N, int64_t H, int64_t I,
                                           int64_t E, int dt) {
  if (!valid_dtype(dt) || N < 0 || N > kMaxRows || H < 1 || I < 1 || E < 1 ||
      E > kMaxDispatchE || H > INT32_MAX || I > INT32_MAX)
    return 0;
  int64_t ei;
  if (!mul_ok(E, I, &ei) || !bytes_ok(ei, H, 4) ||
      !bytes_ok(N, H > I ? H : I, 16))
    return 0;
  return moe::experts_backward_layout(N, H, I, E, dt).total;
}

int moe_experts_backward(const void* xd, int dt, int64_t N, int64_t H,
                         int64_t I, int64_t E, const void* w_gate,
                         const void* w_up, const void* w_down,
                         const uint32_t* offsets, const void* gate,
                         const void* up, const void* act, const void* grad_y,
                         void* grad_xd, float* grad_w_gate, float* grad_w_up,
                         float* grad_w_down, void* workspace,
                         size_t workspace_bytes, void* stream) {
  const char* f = "moe_experts_backward";
  const int s = check_experts(xd, dt, N, H, I, E, w_gate, w_up, w_down,
                              offsets, act, grad_y);
  if (s != MOE_OK) return s;
  if (!grad_w_gate || !grad_w_up || !grad_w_down || !offsets)
    return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", f);
  if (N > 0 && (!gate || !up || !grad_xd))
    return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", f);
  const size_t need = moe_experts_backward_workspace_size(N, H, I, E, dt);
  if (need == 0) return fail(MOE_ERR_SHAPE, "%s: sizes out of range", f);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_INVALID_ARG, "%s: workspace needs %zu bytes", f, need);
  if ((uintptr_t)workspace % 256 != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", f);
  // with no rows every weight gradient is zero, which the kernels write too
  return hip_status(moe::launch_experts_backward(
                        xd, dt, N, H, I, (int)E, w_gate, w_up, w_down,
                        offsets, gate, up, act, grad_y, grad_xd, grad_w_gate,
                        grad_w_up, grad_w_down, workspace,
                        (hipStream_t)stream),
                    f);
}

int moe_dispatch_backward(const void* grad_xd, int dt, int64_t N, int64_t T,
                          int64_t H, int64_t top_k,
                          const uint32_t* token_row, void* grad_x,
                          void* stream) {
  // The combine kernel with unit weights.  check_combine only tests the
  // weights pointer for null, so token_row stands in for it; the launch
  // passes no weights.
  const int s = check_combine(grad_xd, dt, N, T, H, top_k, token_row, dt,
                              token_row, grad_x);
  if (s != MOE_OK) return s;
  if (T == 0) return ok();
  return hip_status(moe::launch_combine(grad_xd, dt, N, T, H, (int)top_k,
                                        nullptr, MOE_F32, token_row, grad_x,
                                        (hipStream_t)stream),
                    "moe_dispatch_backward");
}

}  // extern "C"
