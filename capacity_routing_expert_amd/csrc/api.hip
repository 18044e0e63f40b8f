// C interface of libmoe: argument checks, workspace layout and launch order.  The operations
// and their sources are described in include/moe.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "moe_internal.h"

namespace moe {

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

moe_status device_error(hipError_t err, const char* where) {
  return fail(MOE_ERR_DEVICE, "%s: %s", where, hipGetErrorString(err));
}

// Expert-GEMM kernel timing armed by moe_set_gemm_timing for the next layer or expert-FFN call
// on this thread: up-projection start / stop, down-projection start / stop.
thread_local hipEvent_t g_timing[4] = {nullptr, nullptr, nullptr, nullptr};

// The armed timing events, disarming them; false if none are armed.  A pair (start, stop) of
// a GEMM that is not timed is NULL.
bool take_timing(hipEvent_t (&ev)[4]) {
  if (!g_timing[0] && !g_timing[2]) return false;
  for (int i = 0; i < 4; ++i) {
    ev[i] = g_timing[i];
    g_timing[i] = nullptr;
  }
  return true;
}

// Router and combine kernel timing armed by moe_set_stage_timing for the next layer call on this
// thread: router start / stop, combine start / stop.
thread_local hipEvent_t g_stage_timing[4] = {nullptr, nullptr, nullptr, nullptr};

bool take_stage_timing(hipEvent_t (&ev)[4]) {
  if (!g_stage_timing[0] && !g_stage_timing[2]) return false;
  for (int i = 0; i < 4; ++i) {
    ev[i] = g_stage_timing[i];
    g_stage_timing[i] = nullptr;
  }
  return true;
}

// The events of one GEMM (pair 0: up-projection, 1: down-projection), or NULL if not timed.
const hipEvent_t* timing_pair(bool timed, const hipEvent_t (&ev)[4], int pair) {
  return timed && ev[2 * pair] ? ev + 2 * pair : nullptr;
}

// Records the non-NULL timing events among ev[0 .. n-1] where the stream stands (a GEMM that
// launches nothing).
moe_status record_now(const hipEvent_t* ev, int n, hipStream_t st) {
  for (int i = 0; i < n; ++i)
    if (ev[i])
      if (hipError_t err = hipEventRecord(ev[i], st); err != hipSuccess)
        return device_error(err, "hipEventRecord");
  return MOE_OK;
}

// One timed launch (an expert GEMM, the router or the combine), with its kernel start and stop
// recorded in ev[0], ev[1] when `ev` is given (the events ride on the launch itself); a launch
// that turns out empty records them back to back.
template <typename F>
moe_status run_timed_stage(const hipEvent_t* ev, hipStream_t st, const char* what, F launch) {
  if (ev) arm_launch_events(ev[0], ev[1]);
  const hipError_t err = launch();
  hipEvent_t a, b;
  const bool unused = ev && take_launch_events(&a, &b);  // not taken: nothing was launched
  if (err != hipSuccess) return device_error(err, what);
  return unused ? record_now(ev, 2, st) : MOE_OK;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

moe_status check_shape(const moe_shape* s) {
  if (!s) return fail(MOE_ERR_INVALID_ARGUMENT, "shape is NULL");
  if (s->T < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "T = %lld < 0", (long long)s->T);
  if (s->d_model < 1 || s->d_ff < 1)
    return fail(MOE_ERR_INVALID_ARGUMENT, "d_model = %d, d_ff = %d must be >= 1", s->d_model, s->d_ff);
  if (s->n_experts < 1) return fail(MOE_ERR_INVALID_ARGUMENT, "n_experts = %d < 1", s->n_experts);
  if (s->n_experts > 256)
    return fail(MOE_ERR_INVALID_ARGUMENT, "n_experts = %d > 256", s->n_experts);
  if (s->top_k < 1 || s->top_k > s->n_experts)
    return fail(MOE_ERR_INVALID_ARGUMENT, "top_k = %d not in [1, n_experts = %d]", s->top_k,
                s->n_experts);
  if (s->capacity < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "capacity = %d < 0", s->capacity);
  if (s->T * (int64_t)s->top_k >= ((int64_t)1 << 31))
    return fail(MOE_ERR_UNSUPPORTED, "T * top_k = %lld >= 2^31", (long long)(s->T * s->top_k));
  if (s->dtype != MOE_F32 && s->dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "dtype %d unknown", s->dtype);
  if (s->weight_layout != MOE_WEIGHTS_ROW_MAJOR && s->weight_layout != MOE_WEIGHTS_PACKED)
    return fail(MOE_ERR_INVALID_ARGUMENT, "weight_layout %d unknown", s->weight_layout);
  if (s->weight_layout == MOE_WEIGHTS_PACKED && s->dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "packed weights are bf16 only");
  // a packed expert matrix (up to 2 d_ff x d_model for the gated W13) is addressed with 32-bit
  // byte offsets as a whole
  if (s->weight_layout == MOE_WEIGHTS_PACKED &&
      (int64_t)2 * ((s->d_ff + 31) / 32 * 32) * ((s->d_model + 31) / 32 * 32) * 2 >= ((int64_t)1 << 32))
    return fail(MOE_ERR_UNSUPPORTED, "packed expert weights of %d x %d: 4 GiB or more per expert",
                s->d_ff, s->d_model);
  if (s->dtype == MOE_BF16 && (s->d_model % 8 != 0 || s->d_ff % 8 != 0))
    return fail(MOE_ERR_UNSUPPORTED, "bf16 needs d_model (%d) and d_ff (%d) multiples of 8",
                s->d_model, s->d_ff);
  // the router and the expert GEMMs address x with 32-bit byte offsets
  const int64_t x_bytes = s->T * (int64_t)s->d_model * (s->dtype == MOE_BF16 ? 2 : 4);
  if (x_bytes >= ((int64_t)1 << 31))
    return fail(MOE_ERR_UNSUPPORTED, "x of %lld bytes: must be below 2 GiB", (long long)x_bytes);
  if (s->dtype == MOE_BF16 && (int64_t)256 * (s->d_model > s->d_ff ? s->d_model : s->d_ff) * 2 >=
                                  ((int64_t)1 << 31))
    return fail(MOE_ERR_UNSUPPORTED, "d_model / d_ff too large for 32-bit tile offsets");
  return MOE_OK;
}

size_t elem_bytes(const moe_shape& s) { return s.dtype == MOE_BF16 ? 2 : 4; }

// Data pointers of the dtype: 16-byte alignment for bf16 (vector loads), 4 for fp32.
moe_status check_data_ptr(const moe_shape& s, const void* p, const char* name) {
  if (!p) return fail(MOE_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  const size_t a = s.dtype == MOE_BF16 ? 16 : 4;
  if (!aligned(p, a)) return fail(MOE_ERR_UNSUPPORTED, "%s is not %zu-byte aligned", name, a);
  return MOE_OK;
}

moe_status check_ptr(const void* p, size_t a, const char* name) {
  if (!p) return fail(MOE_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (!aligned(p, a)) return fail(MOE_ERR_UNSUPPORTED, "%s is not %zu-byte aligned", name, a);
  return MOE_OK;
}

moe_status check_ws(const moe_shape& s, const void* ws, size_t ws_bytes,
                    LayoutKind kind = kLayoutCompact) {
  const size_t need = layout(s, kind).total;
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, need);
  if (need && !ws) return fail(MOE_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(MOE_ERR_UNSUPPORTED, "workspace is not 256-byte aligned");
  return MOE_OK;
}

#define MOE_TRY(expr)            \
  do {                           \
    moe_status _st = (expr);     \
    if (_st != MOE_OK) return _st; \
  } while (0)

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

}  // namespace

int64_t max_rows(const moe_shape& s) {
  const int64_t a = s.T * (int64_t)s.top_k;
  const int64_t b = (int64_t)s.n_experts * s.capacity;
  return a < b ? a : b;
}

Workspace layout(const moe_shape& s, LayoutKind kind) {
  Workspace w;
  const int64_t N = s.T * (int64_t)s.top_k;
  const int64_t E = s.n_experts;
  const int64_t nb_a = dispatch_blocks(N), nb_p = dispatch_blocks(N, true), nb_r = dispatch_runs(N);
  const int64_t nb = std::max(nb_a, std::max(nb_p, nb_r));
  const bool padded = kind == kLayoutPadded, dropless = kind == kLayoutDropless;
  const int64_t rows = padded ? E * s.capacity : dropless ? N : max_rows(s);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at_ = o;
    o = align256(o + bytes);
    return at_;
  };
  w.ids = take((size_t)N * 4);
  w.gates = take((size_t)N * 4);
  w.slot_of = take(dropless ? 0 : (size_t)N * 4);
  w.drop = take(dropless ? 0 : (size_t)N);
  w.counts = take((size_t)E * 4);
  w.offsets = take((size_t)(E + 1) * 4);
  w.seg_start = take(dropless ? 0 : (size_t)(E + 2) * 4);
  w.blk_hist = take((size_t)nb * (E + 1) * 4);
  w.keys = take(dropless ? 0 : (size_t)N * 8);  // read in 16-byte pairs up to its 256-B end
  w.rank = take(dropless ? 0 : (size_t)N * 4);
  w.row_token = take((size_t)(dropless ? N : max_rows(s)) * 4);
  w.pairs = take(dropless ? (size_t)N * 4 : 0);
  w.row_token_pad = take(padded ? (size_t)rows * 4 : 0);
  w.offsets_pad = take(padded ? (size_t)(E + 1) * 4 : 0);
  w.h = take((size_t)rows * s.d_ff * elem_bytes(s));
  w.y = take((size_t)rows * s.d_model * elem_bytes(s));
  w.total = o;
  return w;
}

namespace {

moe_status do_route(const moe_shape& s, const void* x, const void* w_router, const float* b_router,
                    int32_t* ids, float* gates, float* logits, hipStream_t st) {
  hipError_t err = launch_route(s, x, w_router, b_router, ids, gates, logits, st);
  return err == hipSuccess ? MOE_OK : device_error(err, "route");
}

moe_status do_dispatch(const moe_shape& s, const int32_t* ids, const float* gates, int32_t* counts,
                       int32_t* offsets, int32_t* slot_of, int32_t* row_token, uint8_t* drop,
                       void* ws, hipStream_t st) {
  const Workspace L = layout(s);
  hipError_t err = launch_dispatch(s, ids, gates, counts, offsets, slot_of, row_token, drop,
                                   at<int32_t>(ws, L.seg_start), at<int32_t>(ws, L.blk_hist),
                                   at<uint64_t>(ws, L.keys), at<int32_t>(ws, L.rank), st);
  return err == hipSuccess ? MOE_OK : device_error(err, "dispatch");
}

moe_status check_forward_args(const moe_shape* shape, const void* x, const void* w_router,
                              const float* b_router, const void* w1, const void* b1,
                              const void* w2, const void* b2, void* out, void* ws,
                              size_t ws_bytes, bool padded = false, bool gated = false) {
  MOE_TRY(check_shape(shape));
  const moe_shape& s = *shape;
  MOE_TRY(check_data_ptr(s, x, "x"));
  MOE_TRY(check_data_ptr(s, w_router, "w_router"));
  if (b_router) MOE_TRY(check_ptr(b_router, 4, "b_router"));
  MOE_TRY(check_data_ptr(s, w1, "w1"));
  if (!gated) MOE_TRY(check_data_ptr(s, b1, "b1"));  // the gated expert has no biases
  MOE_TRY(check_data_ptr(s, w2, "w2"));
  if (!gated) MOE_TRY(check_data_ptr(s, b2, "b2"));
  MOE_TRY(check_data_ptr(s, out, "out"));
  if (out == x) return fail(MOE_ERR_INVALID_ARGUMENT, "out aliases x");
  if (padded && (int64_t)s.n_experts * s.capacity >= ((int64_t)1 << 31))
    return fail(MOE_ERR_UNSUPPORTED, "n_experts * capacity = %lld >= 2^31",
                (long long)((int64_t)s.n_experts * s.capacity));
  MOE_TRY(check_ws(s, ws, ws_bytes, padded ? kLayoutPadded : kLayoutCompact));
  return MOE_OK;
}

moe_status layer_forward(const moe_shape* shape, const void* x, const void* w_router,
                         const float* b_router, const void* w1, const void* b1, const void* w2,
                         const void* b2, void* out, int32_t* topk_ids, float* topk_gates,
                         int32_t* slot_of, uint8_t* drop_mask, int32_t* expert_counts, void* ws,
                         size_t ws_bytes, hipStream_t st, moe_event_t const* events,
                         bool padded = false, void* y_rows = nullptr, bool gated = false) {
  hipEvent_t tev[4], sev[4];
  const bool timed = take_timing(tev);  // both consumed by this call even if it fails
  const bool stimed = take_stage_timing(sev);
  MOE_TRY(check_shape(shape));
  const moe_shape& s = *shape;
  auto rec = [&](int i) -> moe_status {
    if (!events) return MOE_OK;
    hipError_t err = hipEventRecord((hipEvent_t)events[i], st);
    return err == hipSuccess ? MOE_OK : device_error(err, "hipEventRecord");
  };
  if (s.T == 0) {  // empty batch: nothing to check or enqueue
    for (int i = 0; i < 6; ++i) MOE_TRY(rec(i));
    if (stimed) MOE_TRY(record_now(sev, 4, st));
    return timed ? record_now(tev, 4, st) : MOE_OK;
  }
  if (gated) {
    if (s.dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "the gated expert is bf16 only");
    if ((int64_t)4 * s.d_ff * s.d_model >= ((int64_t)1 << 31))
      return fail(MOE_ERR_UNSUPPORTED, "2 * d_ff * d_model bf16 weights per expert: >= 2 GiB");
  }
  MOE_TRY(check_forward_args(shape, x, w_router, b_router, w1, b1, w2, b2, out, ws, ws_bytes,
                             padded, gated));
  if (y_rows) MOE_TRY(check_data_ptr(s, y_rows, "y_rows"));
  if (topk_ids) MOE_TRY(check_ptr(topk_ids, 4, "topk_ids"));
  if (topk_gates) MOE_TRY(check_ptr(topk_gates, 4, "topk_gates"));
  if (slot_of) MOE_TRY(check_ptr(slot_of, 4, "slot_of"));
  if (expert_counts) MOE_TRY(check_ptr(expert_counts, 4, "expert_counts"));
  const Workspace L = layout(s, padded ? kLayoutPadded : kLayoutCompact);
  int32_t* ids = topk_ids ? topk_ids : at<int32_t>(ws, L.ids);
  float* gates = topk_gates ? topk_gates : at<float>(ws, L.gates);
  int32_t* slots = slot_of ? slot_of : at<int32_t>(ws, L.slot_of);
  uint8_t* drop = drop_mask ? drop_mask : at<uint8_t>(ws, L.drop);
  int32_t* counts = expert_counts ? expert_counts : at<int32_t>(ws, L.counts);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* row_token = at<int32_t>(ws, L.row_token);
  void* h = at<void>(ws, L.h);
  void* y = y_rows ? y_rows : at<void>(ws, L.y);
  int64_t rows = max_rows(s);

  MOE_TRY(rec(0));
  MOE_TRY(run_timed_stage(timing_pair(stimed, sev, 0), st, "route", [&] {
    return launch_route(s, x, w_router, b_router, ids, gates, nullptr, st);
  }));
  MOE_TRY(rec(1));
  MOE_TRY(do_dispatch(s, ids, gates, counts, offsets, slots, row_token, drop, ws, st));
  if (padded) {  // every expert's buffer is computed whole: rows e * cap .. (e + 1) * cap - 1
    int32_t* rt_pad = at<int32_t>(ws, L.row_token_pad);
    int32_t* off_pad = at<int32_t>(ws, L.offsets_pad);
    hipError_t err = launch_pad_layout(s, ids, offsets, row_token, slots, rt_pad, off_pad, st);
    if (err != hipSuccess) return device_error(err, "padded layout");
    row_token = rt_pad;
    offsets = off_pad;
    rows = (int64_t)s.n_experts * s.capacity;
  }
  MOE_TRY(rec(2));
  MOE_TRY(run_timed_stage(timing_pair(timed, tev, 0), st, "expert up-projection", [&] {
    return gated ? launch_ffn_up_gated(s, x, row_token, offsets, w1, h, rows, st)
                 : launch_ffn_up(s, x, row_token, offsets, w1, b1, h, rows, st);
  }));
  MOE_TRY(rec(3));
  MOE_TRY(run_timed_stage(timing_pair(timed, tev, 1), st, "expert down-projection", [&] {
    return gated ? launch_ffn_down_nobias(s, h, offsets, w2, y, rows, st)
                 : launch_ffn_down(s, h, offsets, w2, b2, y, rows, st);
  }));
  MOE_TRY(rec(4));
  MOE_TRY(run_timed_stage(timing_pair(stimed, sev, 1), st, "combine",
                          [&] { return launch_combine(s, x, gates, slots, y, out, st); }));
  MOE_TRY(rec(5));
  return MOE_OK;
}

// Dropless pair-order flow: checks shared by the layer call and the expert call.
moe_status check_dropless(const moe_shape& s, bool gated) {
  if (s.dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "the dropless flow is bf16 only");
  // GEMM 2 reads the pair rows of H with 32-bit byte offsets
  if (s.T * (int64_t)s.top_k * s.d_ff * 2 >= ((int64_t)1 << 31))
    return fail(MOE_ERR_UNSUPPORTED, "T * top_k * d_ff bf16 pair activations: >= 2 GiB");
  if (gated && (int64_t)4 * s.d_ff * s.d_model >= ((int64_t)1 << 31))
    return fail(MOE_ERR_UNSUPPORTED, "2 * d_ff * d_model bf16 weights per expert: >= 2 GiB");
  return MOE_OK;
}

moe_status ffn_pairs(const moe_shape& s, const void* x, const int32_t* sorted_pairs,
                     const int32_t* row_token, const int32_t* offsets, const void* w1,
                     const void* b1, const void* w2, const void* b2, const float* weights,
                     bool gated, void* h, void* pair_rows, hipStream_t st,
                     moe_event_t const* events, const hipEvent_t* tev) {
  const int64_t rows = s.T * (int64_t)s.top_k;
  MOE_TRY(run_timed_stage(tev && tev[0] ? tev : nullptr, st,
                          "expert up-projection (pair order)", [&] {
    return launch_ffn_up_pairs(s, x, row_token, sorted_pairs, offsets, w1, gated ? nullptr : b1,
                               h, rows, gated, st);
  }));
  hipError_t err;
  if (events && (err = hipEventRecord((hipEvent_t)events[3], st)) != hipSuccess)
    return device_error(err, "hipEventRecord");
  MOE_TRY(run_timed_stage(tev && tev[2] ? tev + 2 : nullptr, st,
                          "expert down-projection (pair order)", [&] {
    return launch_ffn_down_pairs(s, h, sorted_pairs, offsets, w2, gated ? nullptr : b2, weights,
                                 pair_rows, rows, st);
  }));
  return MOE_OK;
}

moe_status layer_forward_dropless(const moe_shape* shape, const void* x, const void* w_router,
                                  const float* b_router, const void* w1, const void* b1,
                                  const void* w2, const void* b2, bool gated, void* out,
                                  int32_t* topk_ids, float* topk_gates, int32_t* expert_counts,
                                  void* pair_rows, void* ws, size_t ws_bytes, hipStream_t st,
                                  moe_event_t const* events) {
  hipEvent_t tev[4];
  const bool timed = take_timing(tev);  // consumed by this call even if it fails
  MOE_TRY(check_shape(shape));
  const moe_shape& s = *shape;
  if (events)
    for (int i = 0; i < 6; ++i)
      if (!events[i]) return fail(MOE_ERR_INVALID_ARGUMENT, "events[%d] is NULL", i);
  auto rec = [&](int i) -> moe_status {
    if (!events) return MOE_OK;
    hipError_t err = hipEventRecord((hipEvent_t)events[i], st);
    return err == hipSuccess ? MOE_OK : device_error(err, "hipEventRecord");
  };
  if (s.T == 0) {  // empty batch: nothing to check or enqueue
    for (int i = 0; i < 6; ++i) MOE_TRY(rec(i));
    return timed ? record_now(tev, 4, st) : MOE_OK;
  }
  MOE_TRY(check_dropless(s, gated));
  MOE_TRY(check_data_ptr(s, x, "x"));
  MOE_TRY(check_data_ptr(s, w_router, "w_router"));
  if (b_router) MOE_TRY(check_ptr(b_router, 4, "b_router"));
  MOE_TRY(check_data_ptr(s, w1, "w1"));
  MOE_TRY(check_data_ptr(s, w2, "w2"));
  if (!gated) {
    MOE_TRY(check_data_ptr(s, b1, "b1"));
    MOE_TRY(check_data_ptr(s, b2, "b2"));
  }
  MOE_TRY(check_data_ptr(s, out, "out"));
  if (out == x) return fail(MOE_ERR_INVALID_ARGUMENT, "out aliases x");
  if (pair_rows) MOE_TRY(check_data_ptr(s, pair_rows, "pair_rows"));
  if (topk_ids) MOE_TRY(check_ptr(topk_ids, 4, "topk_ids"));
  if (topk_gates) MOE_TRY(check_ptr(topk_gates, 4, "topk_gates"));
  if (expert_counts) MOE_TRY(check_ptr(expert_counts, 4, "expert_counts"));
  MOE_TRY(check_ws(s, ws, ws_bytes, kLayoutDropless));
  const Workspace L = layout(s, kLayoutDropless);
  int32_t* ids = topk_ids ? topk_ids : at<int32_t>(ws, L.ids);
  float* gates = topk_gates ? topk_gates : at<float>(ws, L.gates);
  int32_t* counts = expert_counts ? expert_counts : at<int32_t>(ws, L.counts);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* pairs = at<int32_t>(ws, L.pairs);
  int32_t* row_token = at<int32_t>(ws, L.row_token);
  void* y = pair_rows ? pair_rows : at<void>(ws, L.y);

  MOE_TRY(rec(0));
  MOE_TRY(do_route(s, x, w_router, b_router, ids, gates, nullptr, st));
  MOE_TRY(rec(1));
  hipError_t err = launch_dispatch_pairs(s, ids, counts, offsets, pairs, row_token,
                                         at<int32_t>(ws, L.blk_hist), st);
  if (err != hipSuccess) return device_error(err, "pair dispatch");
  MOE_TRY(rec(2));
  MOE_TRY(ffn_pairs(s, x, pairs, row_token, offsets, w1, b1, w2, b2, gates, gated,
                    at<void>(ws, L.h), y, st, events, timed ? tev : nullptr));  // pairs may be NULL
  MOE_TRY(rec(4));
  err = launch_moe_sum(s, x, ids, y, out, st);
  if (err != hipSuccess) return device_error(err, "moe_sum");
  MOE_TRY(rec(5));
  return MOE_OK;
}

// ---------------------------------------------------------------- batches of a pool
// Workspace of moe_layer_forward_batches: one batch's workspace (reused batch after batch, the
// calls being ordered on one stream), then the pool's buffers.
struct BatchesLayout {
  Workspace per;  // offsets relative to the start of the workspace
  size_t ids, gates, order, x_perm, ids_perm, gates_perm, out_perm, total;
};

moe_shape pool_shape(const moe_shape& b, int32_t n_batches) {
  moe_shape p = b;
  p.T = b.T * (int64_t)n_batches;
  return p;
}

BatchesLayout batches_layout(const moe_shape& b, int32_t n_batches) {
  BatchesLayout w;
  w.per = layout(b);
  const int64_t T = b.T * (int64_t)n_batches;
  const size_t eb = elem_bytes(b), k = (size_t)b.top_k;
  size_t o = w.per.total;
  auto take = [&](size_t bytes) {
    const size_t at_ = o;
    o = align256(o + bytes);
    return at_;
  };
  w.ids = take((size_t)T * k * 4);
  w.gates = take((size_t)T * k * 4);
  w.order = take((size_t)T * 4);
  w.x_perm = take((size_t)T * b.d_model * eb);
  w.ids_perm = take((size_t)T * k * 4);
  w.gates_perm = take((size_t)T * k * 4);
  w.out_perm = take((size_t)T * b.d_model * eb);
  w.total = o;
  return w;
}

// shape and pool checks shared by the scheduling calls; `consolidate` adds the sort's limits
moe_status check_batches(const moe_shape* batch_shape, int32_t n_batches, bool consolidate) {
  MOE_TRY(check_shape(batch_shape));
  const moe_shape& b = *batch_shape;
  if (n_batches < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "n_batches = %d < 0", n_batches);
  const moe_shape p = pool_shape(b, n_batches);
  MOE_TRY(check_shape(&p));  // the pool's T * k and x size limits
  if (consolidate) {
    if (p.T > kSchedMaxT)
      return fail(MOE_ERR_UNSUPPORTED, "a pool of %lld tokens: the scheduler sorts at most %d",
                  (long long)p.T, kSchedMaxT);
    if (b.top_k > kSchedMaxK ||
        b.top_k * schedule_bits_e(b.n_experts) + kSchedIndexBits > 64)
      return fail(MOE_ERR_UNSUPPORTED, "top_k = %d ids of %d experts do not fit a 64-bit key",
                  b.top_k, b.n_experts);
  }
  return MOE_OK;
}

moe_status layer_forward_batches(const moe_shape* batch_shape, int32_t n_batches,
                                 bool consolidate, const void* x, const void* w_router,
                                 const float* b_router, const void* w1, const void* b1,
                                 const void* w2, const void* b2, void* out, int32_t* topk_ids,
                                 float* topk_gates, int32_t* order, int32_t* batch_experts,
                                 void* ws, size_t ws_bytes, hipStream_t st,
                                 moe_event_t const* events) {
  MOE_TRY(check_batches(batch_shape, n_batches, consolidate));
  const moe_shape& bs = *batch_shape;
  if (events)
    for (int i = 0; i < 5; ++i)
      if (!events[i]) return fail(MOE_ERR_INVALID_ARGUMENT, "events[%d] is NULL", i);
  auto rec = [&](int i) -> moe_status {
    if (!events) return MOE_OK;
    hipError_t err = hipEventRecord((hipEvent_t)events[i], st);
    return err == hipSuccess ? MOE_OK : device_error(err, "hipEventRecord");
  };
  const moe_shape ps = pool_shape(bs, n_batches);
  if (ps.T == 0) {  // empty pool: nothing to check or enqueue
    for (int i = 0; i < 5; ++i) MOE_TRY(rec(i));
    return MOE_OK;
  }
  MOE_TRY(check_data_ptr(bs, x, "x"));
  MOE_TRY(check_data_ptr(bs, w_router, "w_router"));
  if (b_router) MOE_TRY(check_ptr(b_router, 4, "b_router"));
  MOE_TRY(check_data_ptr(bs, w1, "w1"));
  MOE_TRY(check_data_ptr(bs, b1, "b1"));
  MOE_TRY(check_data_ptr(bs, w2, "w2"));
  MOE_TRY(check_data_ptr(bs, b2, "b2"));
  MOE_TRY(check_data_ptr(bs, out, "out"));
  if (out == x) return fail(MOE_ERR_INVALID_ARGUMENT, "out aliases x");
  if (topk_ids) MOE_TRY(check_ptr(topk_ids, 4, "topk_ids"));
  if (topk_gates) MOE_TRY(check_ptr(topk_gates, 4, "topk_gates"));
  if (order) MOE_TRY(check_ptr(order, 4, "order"));
  if (batch_experts) MOE_TRY(check_ptr(batch_experts, 4, "batch_experts"));
  const BatchesLayout L = batches_layout(bs, n_batches);
  if (ws_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, L.total);
  if (!ws) return fail(MOE_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(MOE_ERR_UNSUPPORTED, "workspace is not 256-byte aligned");

  const int k = bs.top_k, E = bs.n_experts, B = (int)bs.T;
  const size_t eb = elem_bytes(bs), xrow = (size_t)bs.d_model * eb;
  int32_t* ids = topk_ids ? topk_ids : at<int32_t>(ws, L.ids);
  float* gates = topk_gates ? topk_gates : at<float>(ws, L.gates);
  int32_t* ord = order ? order : at<int32_t>(ws, L.order);
  const Workspace& W = L.per;
  hipError_t err;

  MOE_TRY(rec(0));
  MOE_TRY(do_route(ps, x, w_router, b_router, ids, gates, nullptr, st));  // once for the pool
  MOE_TRY(rec(1));
  const char* xb = static_cast<const char*>(x);
  const int32_t* idsb = ids;
  const float* gb = gates;
  char* outb = static_cast<char*>(out);
  if (consolidate) {
    if ((err = launch_schedule(ids, (int)ps.T, k, E, ord, st)) != hipSuccess)
      return device_error(err, "schedule");
    if ((err = launch_permute_rows(x, ord, at<void>(ws, L.x_perm), ps.T, (int)xrow, false, st)) !=
            hipSuccess ||
        (err = launch_permute_rows(ids, ord, at<void>(ws, L.ids_perm), ps.T, k * 4, false, st)) !=
            hipSuccess ||
        (err = launch_permute_rows(gates, ord, at<void>(ws, L.gates_perm), ps.T, k * 4, false,
                                   st)) != hipSuccess)
      return device_error(err, "batch gather");
    xb = at<char>(ws, L.x_perm);
    idsb = at<int32_t>(ws, L.ids_perm);
    gb = at<float>(ws, L.gates_perm);
    outb = at<char>(ws, L.out_perm);
  }
  if (batch_experts &&
      (err = launch_batch_experts(idsb, nullptr, B, n_batches, k, E, batch_experts, st)) !=
          hipSuccess)
    return device_error(err, "active experts");
  MOE_TRY(rec(2));
  for (int32_t b = 0; b < n_batches; ++b) {  // one batch after the other, as a serving loop runs
    const size_t r0 = (size_t)b * B;
    const int32_t* ib = idsb + r0 * k;
    const float* g = gb + r0 * k;
    MOE_TRY(do_dispatch(bs, ib, g, at<int32_t>(ws, W.counts), at<int32_t>(ws, W.offsets),
                        at<int32_t>(ws, W.slot_of), at<int32_t>(ws, W.row_token),
                        at<uint8_t>(ws, W.drop), ws, st));
    if ((err = launch_ffn_up(bs, xb + r0 * xrow, at<int32_t>(ws, W.row_token),
                             at<int32_t>(ws, W.offsets), w1, b1, at<void>(ws, W.h), max_rows(bs),
                             st)) != hipSuccess)
      return device_error(err, "expert up-projection");
    if ((err = launch_ffn_down(bs, at<void>(ws, W.h), at<int32_t>(ws, W.offsets), w2, b2,
                               at<void>(ws, W.y), max_rows(bs), st)) != hipSuccess)
      return device_error(err, "expert down-projection");
    if ((err = launch_combine(bs, xb + r0 * xrow, g, at<int32_t>(ws, W.slot_of),
                              at<void>(ws, W.y), outb + r0 * xrow, st)) != hipSuccess)
      return device_error(err, "combine");
  }
  MOE_TRY(rec(3));
  if (consolidate &&
      (err = launch_permute_rows(outb, ord, out, ps.T, (int)xrow, true, st)) != hipSuccess)
    return device_error(err, "batch scatter");
  MOE_TRY(rec(4));
  return MOE_OK;
}

// ---------------------------------------------------------------- allocation-free entry point
// The workspace of moe_layer_forward_noalloc: a fixed array in device memory that the library
// holds on every device it runs on until the process ends.  Host code never uses the array's
// own name as an address (on the host that name is only a stand-in); it takes the per-device
// address that hipGetSymbolAddress returns, once per device, with that device current.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the first call on it).
moe_status scratch_address(void** ptr) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return device_error(err, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return device_error(err, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(MOE_ERR_DEVICE, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

int32_t moe_capacity(int64_t T, int32_t top_k, int32_t n_experts, double capacity_factor) {
  if (T < 0 || top_k < 1 || n_experts < 1 || !(capacity_factor >= 0.0) || !isfinite(capacity_factor))
    return -1;
  if (capacity_factor == 0.0 || T == 0) return 0;
  if (T > ((int64_t)1 << 40)) return -1;
  // capacity_factor = m * 2^ex exactly, m a 53-bit integer
  int ex = 0;
  const double mant = frexp(capacity_factor, &ex);
  const int64_t m = (int64_t)ldexp(mant, 53);
  ex -= 53;
  const __int128 num = (__int128)m * T * top_k;  // < 2^53 * 2^40 * 2^31
  if (ex >= 0) return -1;  // C >= 2^52: no capacity of that size fits in int32
  const int sh = -ex;
  // floor(floor(a / 2^sh) / E) = floor(a / (E * 2^sh)) for non-negative integers
  const __int128 q = sh >= 127 ? 0 : (num >> sh) / n_experts;
  if (q > (__int128)INT32_MAX) return -1;
  return (int32_t)q;
}

size_t moe_workspace_bytes(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK) return 0;
  return layout(*shape).total;
}

size_t moe_workspace_bytes_padded(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK) return 0;
  if ((int64_t)shape->n_experts * shape->capacity >= ((int64_t)1 << 31)) return 0;
  return layout(*shape, kLayoutPadded).total;
}

size_t moe_workspace_bytes_dropless(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK) return 0;
  return layout(*shape, kLayoutDropless).total;
}

int64_t moe_max_kept_rows(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK) return -1;
  return max_rows(*shape);
}

size_t moe_packed_weights_bytes(const moe_shape* shape, int32_t rows, int32_t cols) {
  if (check_shape(shape) != MOE_OK || rows < 1 || cols < 1) return 0;
  return (size_t)packed_weight_elems(shape->n_experts, rows, cols) * 2;
}

moe_status moe_pack_weights(const moe_shape* shape, const void* w, int32_t rows, int32_t cols,
                            void* w_packed, moe_stream_t stream) {
  MOE_TRY(check_shape(shape));
  const moe_shape& s = *shape;
  if (s.dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "packed weights are bf16 only");
  if (rows < 1 || cols < 1)
    return fail(MOE_ERR_INVALID_ARGUMENT, "rows = %d, cols = %d must be >= 1", rows, cols);
  if (cols % 8 != 0) return fail(MOE_ERR_UNSUPPORTED, "cols = %d is not a multiple of 8", cols);
  MOE_TRY(check_ptr(w, 16, "w"));
  MOE_TRY(check_ptr(w_packed, 16, "w_packed"));
  const size_t in_bytes = (size_t)s.n_experts * rows * cols * 2;
  const size_t out_bytes = (size_t)packed_weight_elems(s.n_experts, rows, cols) * 2;
  const char* a = static_cast<const char*>(w);
  const char* b = static_cast<const char*>(w_packed);
  if (a < b + out_bytes && b < a + in_bytes)
    return fail(MOE_ERR_INVALID_ARGUMENT, "w_packed overlaps w");
  hipError_t err = launch_pack_weights(w, w_packed, s.n_experts, rows, cols, (hipStream_t)stream);
  return err == hipSuccess ? MOE_OK : device_error(err, "pack weights");
}

const char* moe_status_string(int32_t status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE";
    default: return "MOE_STATUS_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

moe_status moe_route(const moe_shape* shape, const void* x, const void* w_router,
                     const float* b_router, int32_t* topk_ids, float* topk_gates, float* logits,
                     void* ws, size_t ws_bytes, moe_stream_t stream) {
  MOE_TRY(check_shape(shape));
  const moe_shape& s = *shape;
  if (s.T == 0) return MOE_OK;  // empty batch: nothing to check or enqueue
  MOE_TRY(check_data_ptr(s, x, "x"));
  MOE_TRY(check_data_ptr(s, w_router, "w_router"));
  if (b_router) MOE_TRY(check_ptr(b_router, 4, "b_router"));
  MOE_TRY(check_ptr(topk_ids, 4, "topk_ids"));
  MOE_TRY(check_ptr(topk_gates, 4, "topk_gates"));
  if (logits) MOE_TRY(check_ptr(logits, 4, "logits"));
  MOE_TRY(check_ws(s, ws, ws_bytes));
  return do_route(s, x, w_router, b_router, topk_ids, topk_gates, logits, (hipStream_t)stream);
}

moe_status moe_dispatch(const moe_shape* shape, const int32_t* topk_ids, const float* topk_gates,
                        int32_t* expert_counts, int32_t* expert_offsets, int32_t* slot_of,
                        int32_t* row_token, uint8_t* drop_mask, const void* x, void* x_routed,
                        void* ws, size_t ws_bytes, moe_stream_t stream) {
  MOE_TRY(check_shape(shape));
  const moe_shape& s = *shape;
  if (s.T == 0) return MOE_OK;  // empty batch: nothing to check or enqueue
  MOE_TRY(check_ptr(topk_ids, 4, "topk_ids"));
  MOE_TRY(check_ptr(topk_gates, 4, "topk_gates"));
  MOE_TRY(check_ptr(expert_counts, 4, "expert_counts"));
  MOE_TRY(check_ptr(expert_offsets, 4, "expert_offsets"));
  MOE_TRY(check_ptr(slot_of, 4, "slot_of"));
  if (max_rows(s) > 0) MOE_TRY(check_ptr(row_token, 4, "row_token"));
  MOE_TRY(check_ptr(drop_mask, 1, "drop_mask"));
  if (!x != !x_routed)
    return fail(MOE_ERR_INVALID_ARGUMENT, "x and x_routed: both or neither NULL");
  const bool gather = x && max_rows(s) > 0;
  if (gather) {
    MOE_TRY(check_data_ptr(s, x, "x"));
    MOE_TRY(check_data_ptr(s, x_routed, "x_routed"));
    const size_t row = (size_t)s.d_model * elem_bytes(s);
    const char* a = static_cast<const char*>(x);
    const char* b = static_cast<const char*>(x_routed);
    if (a < b + (size_t)max_rows(s) * row && b < a + (size_t)s.T * row)
      return fail(MOE_ERR_INVALID_ARGUMENT, "x_routed overlaps x");
  }
  MOE_TRY(check_ws(s, ws, ws_bytes));
  hipStream_t st = (hipStream_t)stream;
  MOE_TRY(do_dispatch(s, topk_ids, topk_gates, expert_counts, expert_offsets, slot_of, row_token,
                      drop_mask, ws, st));
  if (gather) {
    hipError_t err = launch_gather_rows(s, x, row_token, expert_offsets, x_routed, st);
    if (err != hipSuccess) return device_error(err, "routed rows");
  }
  return MOE_OK;
}

moe_status moe_expert_ffn(const moe_shape* shape, const void* x, const int32_t* row_token,
                          const int32_t* expert_offsets, const void* w1, const void* b1,
                          const void* w2, const void* b2, void* y_rows, void* ws,
                          size_t ws_bytes, moe_stream_t stream) {
  hipEvent_t tev[4];
  const bool timed = take_timing(tev);  // consumed by this call even if it fails
  MOE_TRY(check_shape(shape));
  const moe_shape& s = *shape;
  hipStream_t st = (hipStream_t)stream;
  if (s.T == 0) return timed ? record_now(tev, 4, st) : MOE_OK;  // empty batch
  MOE_TRY(check_data_ptr(s, x, "x"));
  if (max_rows(s) > 0) {
    MOE_TRY(check_ptr(row_token, 4, "row_token"));
    MOE_TRY(check_data_ptr(s, y_rows, "y_rows"));
  }
  MOE_TRY(check_ptr(expert_offsets, 4, "expert_offsets"));
  MOE_TRY(check_data_ptr(s, w1, "w1"));
  MOE_TRY(check_data_ptr(s, b1, "b1"));
  MOE_TRY(check_data_ptr(s, w2, "w2"));
  MOE_TRY(check_data_ptr(s, b2, "b2"));
  MOE_TRY(check_ws(s, ws, ws_bytes));
  if (max_rows(s) == 0) return timed ? record_now(tev, 4, st) : MOE_OK;
  const Workspace L = layout(s);
  void* h = at<void>(ws, L.h);
  MOE_TRY(run_timed_stage(timing_pair(timed, tev, 0), st, "expert up-projection", [&] {
    return launch_ffn_up(s, x, row_token, expert_offsets, w1, b1, h, max_rows(s), st);
  }));
  MOE_TRY(run_timed_stage(timing_pair(timed, tev, 1), st, "expert down-projection", [&] {
    return launch_ffn_down(s, h, expert_offsets, w2, b2, y_rows, max_rows(s), st);
  }));
  return MOE_OK;
}

moe_status moe_combine(const moe_shape* shape, const void* x, const float* topk_gates,
                       const int32_t* slot_of, const void* y_rows, void* out,
                       moe_stream_t stream) {
  MOE_TRY(check_shape(shape));
  const moe_shape& s = *shape;
  if (s.T == 0) return MOE_OK;  // empty batch: nothing to check or enqueue
  MOE_TRY(check_data_ptr(s, x, "x"));
  MOE_TRY(check_ptr(topk_gates, 4, "topk_gates"));
  MOE_TRY(check_ptr(slot_of, 4, "slot_of"));
  if (max_rows(s) > 0) MOE_TRY(check_data_ptr(s, y_rows, "y_rows"));
  MOE_TRY(check_data_ptr(s, out, "out"));
  if (out == x) return fail(MOE_ERR_INVALID_ARGUMENT, "out aliases x");
  hipError_t err = launch_combine(s, x, topk_gates, slot_of, y_rows, out, (hipStream_t)stream);
  return err == hipSuccess ? MOE_OK : device_error(err, "combine");
}

moe_status moe_layer_forward(const moe_shape* shape, const void* x, const void* w_router,
                             const float* b_router, const void* w1, const void* b1,
                             const void* w2, const void* b2, void* out, int32_t* topk_ids,
                             float* topk_gates, int32_t* slot_of, uint8_t* drop_mask,
                             int32_t* expert_counts, void* ws, size_t ws_bytes,
                             moe_stream_t stream) {
  return layer_forward(shape, x, w_router, b_router, w1, b1, w2, b2, out, topk_ids, topk_gates,
                       slot_of, drop_mask, expert_counts, ws, ws_bytes, (hipStream_t)stream,
                       nullptr);
}

moe_status moe_layer_forward_noalloc(const moe_shape* shape, const void* x, const void* w_router,
                                     const float* b_router, const void* w1, const void* b1,
                                     const void* w2, const void* b2, void* out,
                                     int32_t* topk_ids, float* topk_gates, int32_t* slot_of,
                                     uint8_t* drop_mask, int32_t* expert_counts,
                                     moe_stream_t stream) {
  MOE_TRY(check_shape(shape));
  const size_t need = layout(*shape).total;
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE,
                "this shape needs %zu bytes of scratch; the fixed scratch holds %zu bytes "
                "(use moe_layer_forward with a workspace)",
                need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (shape->T > 0) MOE_TRY(scratch_address(&ws));
  return layer_forward(shape, x, w_router, b_router, w1, b1, w2, b2, out, topk_ids, topk_gates,
                       slot_of, drop_mask, expert_counts, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES,
                       (hipStream_t)stream, nullptr);
}

moe_status moe_set_gemm_timing(const moe_event_t* events) {
  if (!events) {
    for (int i = 0; i < 4; ++i) g_timing[i] = nullptr;
    return MOE_OK;
  }
  for (int p = 0; p < 2; ++p)
    if (!events[2 * p] != !events[2 * p + 1])
      return fail(MOE_ERR_INVALID_ARGUMENT, "events[%d] and events[%d]: both or neither NULL",
                  2 * p, 2 * p + 1);
  if (!events[0] && !events[2])
    return fail(MOE_ERR_INVALID_ARGUMENT, "events: no GEMM to time (all four NULL)");
  for (int i = 0; i < 4; ++i) g_timing[i] = (hipEvent_t)events[i];
  return MOE_OK;
}

moe_status moe_set_stage_timing(const moe_event_t* events) {
  if (!events) {
    for (int i = 0; i < 4; ++i) g_stage_timing[i] = nullptr;
    return MOE_OK;
  }
  for (int p = 0; p < 2; ++p)
    if (!events[2 * p] != !events[2 * p + 1])
      return fail(MOE_ERR_INVALID_ARGUMENT, "events[%d] and events[%d]: both or neither NULL",
                  2 * p, 2 * p + 1);
  if (!events[0] && !events[2])
    return fail(MOE_ERR_INVALID_ARGUMENT, "events: no kernel to time (all four NULL)");
  for (int i = 0; i < 4; ++i) g_stage_timing[i] = (hipEvent_t)events[i];
  return MOE_OK;
}

moe_status moe_layer_forward_profiled(const moe_shape* shape, const void* x,
                                      const void* w_router, const float* b_router,
                                      const void* w1, const void* b1, const void* w2,
                                      const void* b2, void* out, int32_t* topk_ids,
                                      float* topk_gates, int32_t* slot_of, uint8_t* drop_mask,
                                      int32_t* expert_counts, void* ws, size_t ws_bytes,
                                      moe_stream_t stream, moe_event_t const* events) {
  if (!events) return fail(MOE_ERR_INVALID_ARGUMENT, "events is NULL");
  for (int i = 0; i < 6; ++i)
    if (!events[i]) return fail(MOE_ERR_INVALID_ARGUMENT, "events[%d] is NULL", i);
  return layer_forward(shape, x, w_router, b_router, w1, b1, w2, b2, out, topk_ids, topk_gates,
                       slot_of, drop_mask, expert_counts, ws, ws_bytes, (hipStream_t)stream,
                       events);
}

moe_status moe_layer_forward_padded(const moe_shape* shape, const void* x, const void* w_router,
                                    const float* b_router, const void* w1, const void* b1,
                                    const void* w2, const void* b2, void* out, int32_t* topk_ids,
                                    float* topk_gates, int32_t* slot_of, uint8_t* drop_mask,
                                    int32_t* expert_counts, void* y_rows, void* ws,
                                    size_t ws_bytes, moe_stream_t stream,
                                    moe_event_t const* events) {
  if (events)
    for (int i = 0; i < 6; ++i)
      if (!events[i]) return fail(MOE_ERR_INVALID_ARGUMENT, "events[%d] is NULL", i);
  return layer_forward(shape, x, w_router, b_router, w1, b1, w2, b2, out, topk_ids, topk_gates,
                       slot_of, drop_mask, expert_counts, ws, ws_bytes, (hipStream_t)stream,
                       events, true, y_rows);
}

moe_status moe_layer_forward_gated(const moe_shape* shape, const void* x, const void* w_router,
                                   const float* b_router, const void* w13, const void* w2,
                                   void* out, int32_t* topk_ids, float* topk_gates,
                                   int32_t* slot_of, uint8_t* drop_mask, int32_t* expert_counts,
                                   void* ws, size_t ws_bytes, moe_stream_t stream,
                                   moe_event_t const* events) {
  if (events)
    for (int i = 0; i < 6; ++i)
      if (!events[i]) return fail(MOE_ERR_INVALID_ARGUMENT, "events[%d] is NULL", i);
  return layer_forward(shape, x, w_router, b_router, w13, nullptr, w2, nullptr, out, topk_ids,
                       topk_gates, slot_of, drop_mask, expert_counts, ws, ws_bytes,
                       (hipStream_t)stream, events, false, nullptr, true);
}

moe_status moe_dispatch_pairs(const moe_shape* shape, const int32_t* topk_ids,
                              int32_t* expert_counts, int32_t* expert_offsets,
                              int32_t* sorted_pairs, int32_t* row_token, void* ws,
                              size_t ws_bytes, moe_stream_t stream) {
  MOE_TRY(check_shape(shape));
  const moe_shape& s = *shape;
  if (s.T == 0) return MOE_OK;  // empty batch: nothing to check or enqueue
  MOE_TRY(check_ptr(topk_ids, 4, "topk_ids"));
  MOE_TRY(check_ptr(expert_counts, 4, "expert_counts"));
  MOE_TRY(check_ptr(expert_offsets, 4, "expert_offsets"));
  MOE_TRY(check_ptr(sorted_pairs, 4, "sorted_pairs"));
  MOE_TRY(check_ptr(row_token, 4, "row_token"));
  MOE_TRY(check_ws(s, ws, ws_bytes, kLayoutDropless));
  const Workspace L = layout(s, kLayoutDropless);
  hipError_t err = launch_dispatch_pairs(s, topk_ids, expert_counts, expert_offsets, sorted_pairs,
                                         row_token, at<int32_t>(ws, L.blk_hist),
                                         (hipStream_t)stream);
  return err == hipSuccess ? MOE_OK : device_error(err, "pair dispatch");
}

moe_status moe_expert_ffn_pairs(const moe_shape* shape, const void* x,
                                const int32_t* sorted_pairs, const int32_t* row_token,
                                const int32_t* expert_offsets, const void* w1, const void* b1,
                                const void* w2, const void* b2, const float* topk_weights,
                                int32_t gated, void* pair_rows, void* ws, size_t ws_bytes,
                                moe_stream_t stream) {
  hipEvent_t tev[4];
  const bool timed = take_timing(tev);  // consumed by this call even if it fails
  MOE_TRY(check_shape(shape));
  const moe_shape& s = *shape;
  if (s.T == 0) return timed ? record_now(tev, 4, (hipStream_t)stream) : MOE_OK;
  MOE_TRY(check_dropless(s, gated != 0));
  MOE_TRY(check_data_ptr(s, x, "x"));
  MOE_TRY(check_ptr(sorted_pairs, 4, "sorted_pairs"));
  MOE_TRY(check_ptr(row_token, 4, "row_token"));
  MOE_TRY(check_ptr(expert_offsets, 4, "expert_offsets"));
  MOE_TRY(check_data_ptr(s, w1, "w1"));
  MOE_TRY(check_data_ptr(s, w2, "w2"));
  if (!gated) {
    MOE_TRY(check_data_ptr(s, b1, "b1"));
    MOE_TRY(check_data_ptr(s, b2, "b2"));
  }
  MOE_TRY(check_ptr(topk_weights, 4, "topk_weights"));
  MOE_TRY(check_data_ptr(s, pair_rows, "pair_rows"));
  MOE_TRY(check_ws(s, ws, ws_bytes, kLayoutDropless));
  const Workspace L = layout(s, kLayoutDropless);
  return ffn_pairs(s, x, sorted_pairs, row_token, expert_offsets, w1, b1, w2, b2, topk_weights,
                   gated != 0, at<void>(ws, L.h), pair_rows, (hipStream_t)stream, nullptr,
                   timed ? tev : nullptr);
}

moe_status moe_sum(const moe_shape* shape, const void* x, const int32_t* topk_ids,
                   const void* pair_rows, void* out, moe_stream_t stream) {
  MOE_TRY(check_shape(shape));
  const moe_shape& s = *shape;
  if (s.T == 0) return MOE_OK;  // empty batch: nothing to check or enqueue
  if (x) MOE_TRY(check_data_ptr(s, x, "x"));
  if (topk_ids) MOE_TRY(check_ptr(topk_ids, 4, "topk_ids"));
  MOE_TRY(check_data_ptr(s, pair_rows, "pair_rows"));
  MOE_TRY(check_data_ptr(s, out, "out"));
  if (out == x) return fail(MOE_ERR_INVALID_ARGUMENT, "out aliases x");
  if (out == pair_rows) return fail(MOE_ERR_INVALID_ARGUMENT, "out aliases pair_rows");
  hipError_t err = launch_moe_sum(s, x, topk_ids, pair_rows, out, (hipStream_t)stream);
  return err == hipSuccess ? MOE_OK : device_error(err, "moe_sum");
}

moe_status moe_layer_forward_dropless(const moe_shape* shape, const void* x,
                                      const void* w_router, const float* b_router,
                                      const void* w1, const void* b1, const void* w2,
                                      const void* b2, void* out, int32_t* topk_ids,
                                      float* topk_gates, int32_t* expert_counts, void* pair_rows,
                                      void* ws, size_t ws_bytes, moe_stream_t stream,
                                      moe_event_t const* events) {
  return layer_forward_dropless(shape, x, w_router, b_router, w1, b1, w2, b2, false, out,
                                topk_ids, topk_gates, expert_counts, pair_rows, ws, ws_bytes,
                                (hipStream_t)stream, events);
}

moe_status moe_layer_forward_dropless_gated(const moe_shape* shape, const void* x,
                                            const void* w_router, const float* b_router,
                                            const void* w13, const void* w2, void* out,
                                            int32_t* topk_ids, float* topk_gates,
                                            int32_t* expert_counts, void* pair_rows, void* ws,
                                            size_t ws_bytes, moe_stream_t stream,
                                            moe_event_t const* events) {
  return layer_forward_dropless(shape, x, w_router, b_router, w13, nullptr, w2, nullptr, true,
                                out, topk_ids, topk_gates, expert_counts, pair_rows, ws,
                                ws_bytes, (hipStream_t)stream, events);
}

size_t moe_workspace_bytes_batches(const moe_shape* batch_shape, int32_t n_batches) {
  if (check_batches(batch_shape, n_batches, false) != MOE_OK) return 0;
  return batches_layout(*batch_shape, n_batches).total;
}

moe_status moe_schedule_batches(const moe_shape* batch_shape, int32_t n_batches,
                                const int32_t* topk_ids, int32_t* order,
                                int32_t* batch_experts, int32_t* orig_batch_experts,
                                moe_stream_t stream) {
  MOE_TRY(check_batches(batch_shape, n_batches, true));
  const moe_shape& bs = *batch_shape;
  const int64_t T = bs.T * (int64_t)n_batches;
  if (T == 0) return MOE_OK;  // empty pool: nothing to check or enqueue
  MOE_TRY(check_ptr(topk_ids, 4, "topk_ids"));
  MOE_TRY(check_ptr(order, 4, "order"));
  if (batch_experts) MOE_TRY(check_ptr(batch_experts, 4, "batch_experts"));
  if (orig_batch_experts) MOE_TRY(check_ptr(orig_batch_experts, 4, "orig_batch_experts"));
  hipStream_t st = (hipStream_t)stream;
  const int k = bs.top_k, E = bs.n_experts, B = (int)bs.T;
  hipError_t err = launch_schedule(topk_ids, (int)T, k, E, order, st);
  if (err != hipSuccess) return device_error(err, "schedule");
  if (orig_batch_experts &&
      (err = launch_batch_experts(topk_ids, nullptr, B, n_batches, k, E, orig_batch_experts,
                                  st)) != hipSuccess)
    return device_error(err, "active experts");
  if (batch_experts &&  // the new batches, read through the order
      (err = launch_batch_experts(topk_ids, order, B, n_batches, k, E, batch_experts, st)) !=
          hipSuccess)
    return device_error(err, "active experts");
  return MOE_OK;
}

moe_status moe_layer_forward_batches(const moe_shape* batch_shape, int32_t n_batches,
                                     int32_t consolidate, const void* x, const void* w_router,
                                     const float* b_router, const void* w1, const void* b1,
                                     const void* w2, const void* b2, void* out,
                                     int32_t* topk_ids, float* topk_gates, int32_t* order,
                                     int32_t* batch_experts, void* ws, size_t ws_bytes,
                                     moe_stream_t stream, moe_event_t const* events) {
  return layer_forward_batches(batch_shape, n_batches, consolidate != 0, x, w_router, b_router,
                               w1, b1, w2, b2, out, topk_ids, topk_gates, order, batch_experts,
                               ws, ws_bytes, (hipStream_t)stream, events);
}

}  // extern "C"
