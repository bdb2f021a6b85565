// C-ABI host layer of libmoe: argument checks, workspace layout, kernel choice, launches.
// The operations are those of include/moe.h (see the citations there); nothing here touches data:
// every step of the layer runs in the kernels of this directory.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <string>

#include "kernels.h"
#include "moe.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return MOE_OK;
}

int device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MOE_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// Optional per-kernel timing (moe_profile_events): events[2i] / events[2i+1] are recorded on the
// call's stream before / after its i-th kernel launch.
constexpr int kMaxProfiled = 32;
struct Profile {
  void* const* events = nullptr;
  int n_events = 0;
  int count = 0;
  const char* names[kMaxProfiled] = {};
};
thread_local Profile g_prof;

void prof_reset() { g_prof.count = 0; }

template <class F>
hipError_t timed(const char* name, hipStream_t s, F&& launch) {
  Profile& p = g_prof;
  const int i = p.count;
  const bool on = p.events != nullptr && i < kMaxProfiled && 2 * i + 1 < p.n_events;
  if (on) {
    hipError_t e = hipEventRecord(static_cast<hipEvent_t>(p.events[2 * i]), s);
    if (e != hipSuccess) return e;
  }
  hipError_t e = launch();
  if (on) {
    if (e == hipSuccess) e = hipEventRecord(static_cast<hipEvent_t>(p.events[2 * i + 1]), s);
    p.names[i] = name;
    p.count = i + 1;
  }
  return e;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Carves aligned sub-buffers out of the caller's workspace (or just measures when base is null).
struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <class T>
  T* take(int64_t count) {
    T* p = base ? reinterpret_cast<T*>(base + used) : nullptr;
    used += align_up((size_t)(count > 0 ? count : 0) * sizeof(T));
    return p;
  }
};

constexpr int kMaxExperts = 512;
constexpr int kMaxTopK = 64;
constexpr int kMaxGroups = 4096;

int check_config(const moe_config* c) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "config is NULL");
  if (c->hidden_size <= 0 || c->moe_intermediate_size <= 0 || c->n_routed_experts <= 0 || c->top_k <= 0)
    return fail(MOE_ERR_INVALID_ARG, "sizes must be positive (H=%d I=%d E=%d K=%d)", c->hidden_size,
                c->moe_intermediate_size, c->n_routed_experts, c->top_k);
  if (c->top_k > c->n_routed_experts)
    return fail(MOE_ERR_INVALID_ARG, "top_k (%d) > n_routed_experts (%d)", c->top_k, c->n_routed_experts);
  if (c->n_shared_experts < 0) return fail(MOE_ERR_INVALID_ARG, "n_shared_experts < 0");
  if (c->n_group != 1 || c->topk_group != 1)
    return fail(MOE_ERR_UNSUPPORTED, "only n_group = topk_group = 1 (router without expert groups) is supported");
  if (c->norm_topk_prob != 1) return fail(MOE_ERR_UNSUPPORTED, "only norm_topk_prob = 1 is supported");
  if (c->n_shared_experts > 1) return fail(MOE_ERR_UNSUPPORTED, "at most one shared expert is supported");
  if (c->hidden_size % 128 || c->moe_intermediate_size % 128)
    return fail(MOE_ERR_UNSUPPORTED, "hidden_size and moe_intermediate_size must be multiples of 128");
  if (c->n_routed_experts > kMaxExperts) return fail(MOE_ERR_UNSUPPORTED, "n_routed_experts > %d", kMaxExperts);
  if (c->top_k > kMaxTopK) return fail(MOE_ERR_UNSUPPORTED, "top_k > %d", kMaxTopK);
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "dtype %d", c->dtype);
  if (!(c->routed_scaling_factor == c->routed_scaling_factor)) return fail(MOE_ERR_INVALID_ARG, "scale is NaN");
  return MOE_OK;
}

int check_tokens(int64_t T, const moe_config* c) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "negative token count");
  const int64_t rows = T * (c->top_k + 1);
  if (rows > 0x7fffffffLL) return fail(MOE_ERR_UNSUPPORTED, "T*(K+1) exceeds 2^31-1");
  return MOE_OK;
}

size_t elem_bytes(int dtype) { return dtype == MOE_BF16 ? 2 : 4; }

// The bf16 MFMA kernels address each operand matrix as a uniform base plus a 32-bit per-lane byte
// offset, so every matrix they read must span less than 4 GiB.
int check_span(const char* what, int64_t bytes) {
  if (bytes >= (int64_t(1) << 32))
    return fail(MOE_ERR_UNSUPPORTED, "%s spans %lld bytes; bf16 operands must stay below 4 GiB", what,
                (long long)bytes);
  return MOE_OK;
}

// Operand spans of a bf16 forward over T tokens (x, the intermediate h, one expert's weights).
int check_forward_spans(const moe_config* c, int64_t T) {
  if (c->dtype != MOE_BF16) return MOE_OK;
  const int64_t H = c->hidden_size, I = c->moe_intermediate_size;
  const int64_t rows = T * (c->top_k + c->n_shared_experts);
  int st;
  if ((st = check_span("x [T, H]", T * H * 2))) return st;
  if ((st = check_span("h [rows, I]", rows * I * 2))) return st;
  if ((st = check_span("an expert weight [I, H]", I * H * 2))) return st;
  return check_span("w_router [E, H]", (int64_t)c->n_routed_experts * H * 2);
}

bool use_stream_kernels(int64_t max_rows, int G) { return max_rows <= 4LL * G; }

// bf16 calls of at most 64 rows in all that the stream kernels do not take: the skinny kernels.
bool use_skinny_kernels(const moe_config* c, int64_t max_rows, int G) {
  return c->dtype == MOE_BF16 && !use_stream_kernels(max_rows, G) &&
         moe::skinny_ok(max_rows, c->hidden_size, c->moe_intermediate_size);
}

// Grouped SwiGLU scratch: h, the plan, and the down GEMM's K-range partial sums when it splits K.
struct SwigluWs {
  void* h;
  moe::Groups g;
  float* part;
};

// Plan buffers of G groups over at most max_rows rows.
moe::Groups carve_plan(Carver& cv, int G, int64_t max_rows, int tile_m = moe::kTileM) {
  moe::Groups g;
  g.n_groups = G;
  g.max_rows = max_rows;
  g.tile_m = tile_m;
  g.stream_rows = G >= moe::kStreamMinGroups ? moe::kStreamRows : 0;
  g.max_tiles = (int32_t)((max_rows + tile_m - 1) / tile_m + G);
  g.active = cv.take<int32_t>(G);
  g.counters = cv.take<int32_t>(3);
  g.tiles = cv.take<int32_t>(2LL * g.max_tiles);
  return g;
}

SwigluWs carve_swiglu(Carver& cv, const moe_config* c, int G, int64_t max_rows) {
  SwigluWs w{};
  w.h = cv.take<char>(max_rows * c->moe_intermediate_size * (int64_t)elem_bytes(c->dtype));
  w.g = carve_plan(cv, G, max_rows);
  w.part = nullptr;
  if (c->dtype == MOE_BF16 && !use_stream_kernels(max_rows, G)) {
    const int H = c->hidden_size, I = c->moe_intermediate_size;
    const bool skinny = use_skinny_kernels(c, max_rows, G);
    const int split = skinny ? moe::skinny_down_plan(G, max_rows, H, I).ks : moe::down_tile_ksplit(max_rows, G, H, I);
    if (split > 1) w.part = cv.take<float>((int64_t)split * max_rows * H);
  }
  return w;
}

// Launch the plan (unless the permutation launch already made it) + both grouped GEMMs.
hipError_t run_swiglu(const moe_config* c, const moe::Groups& g, const moe::Weights& w, const void* x, void* h,
                      float* part, const float* row_scale, void* y_rows, bool y_bf16, hipStream_t s,
                      bool planned = false) {
  const int H = c->hidden_size, I = c->moe_intermediate_size;
  if (use_skinny_kernels(c, g.max_rows, g.n_groups)) {
    // the skinny kernels read the group offsets themselves: no plan
    hipError_t e = timed("gateup_skinny", s, [&] {
      return moe::launch_gateup_skinny_bf16(g, w, static_cast<const uint16_t*>(x), static_cast<uint16_t*>(h), H, I,
                                            s);
    });
    if (e != hipSuccess) return e;
    return timed("down_skinny", s, [&] {
      return moe::launch_down_skinny_bf16(g, w, static_cast<const uint16_t*>(h), y_rows, y_bf16, row_scale, part, H,
                                          I, s);
    });
  }
  hipError_t e = planned ? hipSuccess : timed("plan", s, [&] { return moe::launch_plan(g, s); });
  if (e != hipSuccess) return e;
  if (c->dtype == MOE_F32) {
    e = timed("gateup_f32", s, [&] {
      return moe::launch_gateup_f32(g, w, static_cast<const float*>(x), static_cast<float*>(h), H, I, s);
    });
    if (e != hipSuccess) return e;
    return timed("down_f32", s, [&] {
      return moe::launch_down_f32(g, w, static_cast<const float*>(h), static_cast<float*>(y_rows), row_scale, H, I, s);
    });
  }
  // decode-like: every group on the weight-stream kernels; otherwise the groups in the tile list on
  // the tile kernels and, when the plan leaves the small ones out of it, those on the stream kernels
  const bool all_stream = use_stream_kernels(g.max_rows, g.n_groups);
  const bool small_stream = !all_stream && g.stream_rows > 0;
  if (all_stream || small_stream) {
    e = timed("gateup_stream", s, [&] {
      return moe::launch_gateup_stream_bf16(g, w, static_cast<const uint16_t*>(x), static_cast<uint16_t*>(h), H, I,
                                            small_stream, s);
    });
    if (e != hipSuccess) return e;
  }
  if (all_stream)
    return timed("down_stream", s, [&] {
      return moe::launch_down_stream_bf16(g, w, static_cast<const uint16_t*>(h), y_rows, y_bf16, row_scale, H, I,
                                          false, s);
    });
  e = timed("gateup_tile", s, [&] {
    return moe::launch_gateup_tile_bf16(g, w, static_cast<const uint16_t*>(x), static_cast<uint16_t*>(h), H, I, s);
  });
  if (e != hipSuccess) return e;
  if (small_stream) {
    e = timed("down_stream", s, [&] {
      return moe::launch_down_stream_bf16(g, w, static_cast<const uint16_t*>(h), y_rows, y_bf16, row_scale, H, I,
                                          true, s);
    });
    if (e != hipSuccess) return e;
  }
  return timed("down_tile", s, [&] {
    return moe::launch_down_tile_bf16(g, w, static_cast<const uint16_t*>(h), y_rows, y_bf16, row_scale, part, H, I,
                                      s);
  });
}

// Workspace of the full forward (router optional).
struct ForwardWs {
  int32_t* ids;
  float* weights;
  float* router_part;
  int32_t* offsets;
  int32_t* row_token;
  int32_t* pair_row;
  int32_t* perm_scratch;
  SwigluWs sw;
  void* y_rows;
};

ForwardWs carve_forward(Carver& cv, const moe_config* c, int64_t T, bool with_router) {
  const int H = c->hidden_size, E = c->n_routed_experts, K = c->top_k;
  const bool shared = c->n_shared_experts == 1;
  const int64_t P = T * K;
  const int64_t rows = P + (shared ? T : 0);
  const int G = E + (shared ? 1 : 0);
  ForwardWs w{};
  w.ids = cv.take<int32_t>(P);
  w.weights = cv.take<float>(P);
  w.router_part = with_router ? cv.take<float>((int64_t)moe::router_nsplit(T, H, E, c->dtype == MOE_BF16) * T * E)
                              : nullptr;
  w.offsets = cv.take<int32_t>(E + 2);
  w.row_token = cv.take<int32_t>(rows);
  w.pair_row = cv.take<int32_t>(P);
  w.perm_scratch = cv.take<int32_t>(moe::permute_scratch_ints(P, E));
  w.sw = carve_swiglu(cv, c, G, rows);
  w.y_rows = cv.take<char>(rows * H * (int64_t)elem_bytes(c->dtype));
  return w;
}

int run_after_routing(const moe_config* c, int64_t T, const void* x, const int32_t* ids, const float* weights,
                      const void* w_gate, const void* w_up, const void* w_down, const void* ws_gate,
                      const void* ws_up, const void* ws_down, void* y, ForwardWs& w, hipStream_t s) {
  const int H = c->hidden_size, E = c->n_routed_experts, K = c->top_k;
  const bool shared = c->n_shared_experts == 1;
  const int64_t P = T * K;
  moe::Groups g = w.sw.g;
  g.group_offsets = w.offsets;
  g.row_index = w.row_token;
  const bool fused = moe::permute_plan_fused(P, E, g.n_groups);
  hipError_t e = timed(fused ? "permute_plan" : "permute", s, [&] {
    return fused ? moe::launch_permute_plan(ids, T, K, E, w.offsets, w.row_token, w.pair_row, shared, g, nullptr,
                                            nullptr, H, s)
                 : moe::launch_permute(ids, T, K, E, w.offsets, w.row_token, w.pair_row, w.perm_scratch, shared, s);
  });
  if (e != hipSuccess) return device_status(e, "permute");
  moe::Weights wt;
  wt.gate = w_gate;
  wt.up = w_up;
  wt.down = w_down;
  if (shared) {
    wt.s_gate = ws_gate;
    wt.s_up = ws_up;
    wt.s_down = ws_down;
    wt.shared_group = E;
  }
  const bool rows_bf16 = c->dtype == MOE_BF16;
  e = run_swiglu(c, g, wt, x, w.sw.h, w.sw.part, nullptr, w.y_rows, rows_bf16, s, fused);
  if (e != hipSuccess) return device_status(e, "grouped swiglu");
  const char* yr = static_cast<const char*>(w.y_rows);
  const void* ysh = shared ? yr + P * H * (int64_t)elem_bytes(c->dtype) : nullptr;
  e = timed("combine", s, [&] {
    return moe::launch_combine(w.y_rows, rows_bf16, w.pair_row, weights, ysh, y, c->dtype == MOE_BF16, T, K, H, s);
  });
  if (e != hipSuccess) return device_status(e, "combine");
  return ok();
}

// Workspace of the forward with quantized routed experts.  h holds f16 rows for the routed pairs and
// bf16 rows for the shared expert's rows after them; y_rows is bf16.
struct QuantWs {
  int32_t* ids;
  float* weights;
  float* router_part;
  int32_t* offsets;
  int32_t* row_token;
  int32_t* pair_row;
  int32_t* perm_scratch;
  uint16_t* x16;
  uint16_t* h;
  moe::Groups routed;
  void* y_rows;
};

// Whether a quantized forward runs its larger groups on the tile kernels (many rows per group); their
// plan then also lists the shared expert's rows, as group E.
bool quant_tiles(const moe_config* c, moe::QFormat f, int64_t T) {
  const bool shared = c->n_shared_experts == 1;
  const int64_t rows = T * c->top_k + (shared ? T : 0);
  return moe::tile_quant_shape_ok(f, c->hidden_size, c->moe_intermediate_size) &&
         !use_stream_kernels(rows, c->n_routed_experts + (shared ? 1 : 0));
}

QuantWs carve_quant(Carver& cv, const moe_config* c, int64_t T, moe::QFormat f) {
  const int H = c->hidden_size, I = c->moe_intermediate_size, E = c->n_routed_experts, K = c->top_k;
  const bool shared = c->n_shared_experts == 1;
  const int64_t P = T * K;
  const int64_t rows = P + (shared ? T : 0);
  const bool tiles = quant_tiles(c, f, T);
  QuantWs w{};
  w.ids = cv.take<int32_t>(P);
  w.weights = cv.take<float>(P);
  w.router_part = cv.take<float>((int64_t)moe::router_nsplit(T, H, E, true) * T * E);
  w.offsets = cv.take<int32_t>(E + 2);
  w.row_token = cv.take<int32_t>(rows);
  w.pair_row = cv.take<int32_t>(P);
  w.perm_scratch = cv.take<int32_t>(moe::permute_scratch_ints(P, E));
  w.x16 = cv.take<uint16_t>(T * H);
  w.h = cv.take<uint16_t>(rows * I);
  const int tile_m = f == moe::QFormat::kInt4 ? moe::kTileMQ4 : moe::kTileMFp8;
  w.routed = tiles ? carve_plan(cv, E + (shared ? 1 : 0), rows, tile_m) : carve_plan(cv, E, P);
  w.y_rows = cv.take<uint16_t>(rows * H);
  return w;
}

int check_config_quant(const moe_config* c, moe::QFormat f) {
  const bool q4 = f == moe::QFormat::kInt4;
  if (c->dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "%s routed experts need dtype MOE_BF16", q4 ? "4-bit" : "FP8");
  if (!moe::qshape_ok(f, c->hidden_size, c->moe_intermediate_size))
    return fail(MOE_ERR_UNSUPPORTED,
                q4 ? "4-bit routed experts need hidden_size and moe_intermediate_size multiples of 256"
                   : "FP8 routed experts need hidden_size and moe_intermediate_size multiples of 128, at most 8192");
  return MOE_OK;
}

// Operands the kernels move 16 bytes at a time (token rows, weights, codes, 4-bit scales, outputs)
// must start on a 16-byte boundary, index, weight and fp32-scale vectors on a 4-byte one.  NULL
// pointers pass (their presence is checked separately).
struct Aligned {
  const void* p;
  size_t bytes;
  const char* what;
};
int check_aligned(const char* fn, std::initializer_list<Aligned> list) {
  for (const Aligned& a : list)
    if (a.p && reinterpret_cast<uintptr_t>(a.p) % a.bytes)
      return fail(MOE_ERR_INVALID_ARG, "%s: %s must be %zu-byte aligned", fn, a.what, a.bytes);
  return MOE_OK;
}

hipError_t run_router(const moe_config* c, int64_t T, const void* x, const void* w_router, float* part,
                      hipStream_t s) {
  const int H = c->hidden_size, E = c->n_routed_experts;
  if (c->dtype == MOE_BF16)
    return timed("router_logits", s, [&] {
      return moe::launch_router_logits_bf16(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_router),
                                            part, T, H, E, s);
    });
  return timed("router_logits_f32", s, [&] {
    return moe::launch_router_logits_f32(static_cast<const float*>(x), static_cast<const float*>(w_router), part, T,
                                         H, E, s);
  });
}

int check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return MOE_OK;
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (have < need) return fail(MOE_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", have, need);
  if (reinterpret_cast<uintptr_t>(ws) % kAlign)
    return fail(MOE_ERR_WORKSPACE, "workspace must be %zu-byte aligned", kAlign);
  return MOE_OK;
}

// The layer with quantized routed experts (either format): name prefixes the error messages.
int forward_quant(const char* name, const moe_config* cfg, int64_t T, const void* x, const void* w_router,
                  const float* score_bias, const float* logit_offset, const moe::QWeights& qw, const void* ws_gate,
                  const void* ws_up, const void* ws_down, void* y, int32_t* topk_ids_out, float* topk_weights_out,
                  void* workspace, size_t workspace_bytes, void* stream) {
  prof_reset();
  int st = check_config(cfg);
  if (st) return st;
  if ((st = check_config_quant(cfg, qw.format))) return st;
  if ((st = check_tokens(T, cfg))) return st;
  if (T == 0) return ok();
  if (!x || !w_router || !qw.gate_codes || !qw.gate_scales || !qw.up_codes || !qw.up_scales || !qw.down_codes ||
      !qw.down_scales || !y)
    return fail(MOE_ERR_INVALID_ARG, "%s: x, w_router, expert codes and scales and y are required", name);
  const bool shared = cfg->n_shared_experts == 1;
  if (shared && (!ws_gate || !ws_up || !ws_down))
    return fail(MOE_ERR_INVALID_ARG, "%s: shared expert weights are required", name);
  const size_t sa = qw.format == moe::QFormat::kInt4 ? 16 : 4;  // 4-bit scales are read 16 bytes at a time
  if ((st = check_aligned(name, {{x, 16, "x"}, {w_router, 16, "w_router"}, {qw.gate_codes, 16, "gate_codes"},
                                 {qw.up_codes, 16, "up_codes"}, {qw.down_codes, 16, "down_codes"},
                                 {qw.gate_scales, sa, "gate_scales"}, {qw.up_scales, sa, "up_scales"},
                                 {qw.down_scales, sa, "down_scales"}, {ws_gate, 16, "ws_gate"}, {ws_up, 16, "ws_up"},
                                 {ws_down, 16, "ws_down"}, {y, 16, "y"}, {score_bias, 4, "score_bias"},
                                 {logit_offset, 4, "logit_offset"}, {topk_ids_out, 4, "topk_ids_out"},
                                 {topk_weights_out, 4, "topk_weights_out"}})))
    return st;
  if ((st = check_forward_spans(cfg, T))) return st;
  const int H = cfg->hidden_size, I = cfg->moe_intermediate_size, E = cfg->n_routed_experts, K = cfg->top_k;
  const int64_t P = T * K;
  Carver cv(workspace);
  QuantWs w = carve_quant(cv, cfg, T, qw.format);
  if ((st = check_ws(workspace, workspace_bytes, cv.used))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* ids = topk_ids_out ? topk_ids_out : w.ids;
  float* weights = topk_weights_out ? topk_weights_out : w.weights;

  hipError_t e = run_router(cfg, T, x, w_router, w.router_part, s);
  if (e != hipSuccess) return device_status(e, "router logits");
  e = timed("topk", s, [&] {
    return moe::launch_topk(w.router_part, moe::router_nsplit(T, H, E, true), logit_offset, score_bias, T, E, K,
                            cfg->routed_scaling_factor, ids, weights, s);
  });
  if (e != hipSuccess) return device_status(e, "top-k");
  // routed experts: groups 0..E-1 over rows [0, P); the shared expert (bf16) runs in the same
  // launches over rows [P, P + T) (row P + t is token t).  With many rows per group (FP8) the plan
  // lists the shared rows as group E too, and the tile kernels take every group of more than
  // stream_rows rows, the stream kernels the others.
  moe::Groups gr = w.routed;
  gr.group_offsets = w.offsets;
  gr.row_index = w.row_token;
  const bool fused = moe::permute_plan_fused(P, E, gr.n_groups);
  if (fused) {
    e = timed("permute_plan", s, [&] {
      return moe::launch_permute_plan(ids, T, K, E, w.offsets, w.row_token, w.pair_row, shared, gr,
                                      static_cast<const uint16_t*>(x), w.x16, H, s);
    });
    if (e != hipSuccess) return device_status(e, "permute");
  } else {
    e = timed("permute", s, [&] {
      return moe::launch_permute(ids, T, K, E, w.offsets, w.row_token, w.pair_row, w.perm_scratch, shared, s);
    });
    if (e != hipSuccess) return device_status(e, "permute");
    e = timed("f16_rows", s, [&] {
      return moe::launch_f16_rows(static_cast<const uint16_t*>(x), w.x16, T, H, s);
    });
    if (e != hipSuccess) return device_status(e, "f16 rows");
  }
  moe::SharedBf16 sh;
  sh.offsets = w.offsets + E;
  sh.row_index = w.row_token;
  sh.gate = static_cast<const uint16_t*>(ws_gate);
  sh.up = static_cast<const uint16_t*>(ws_up);
  sh.down = static_cast<const uint16_t*>(ws_down);
  sh.x = static_cast<const uint16_t*>(x);
  sh.x_rows = T;
  sh.h = w.h;
  sh.h_rows = P + T;
  const moe::SharedBf16* shp = shared ? &sh : nullptr;
  uint16_t* y_rows = static_cast<uint16_t*>(w.y_rows);
  if (!fused) e = timed("plan", s, [&] { return moe::launch_plan(gr, s); });
  const bool q4 = qw.format == moe::QFormat::kInt4;
  if (quant_tiles(cfg, qw.format, T)) {
    moe::Weights wsh;  // the shared expert's bf16 weights for its tiles
    if (shared) {
      wsh.s_gate = ws_gate;
      wsh.s_up = ws_up;
      wsh.s_down = ws_down;
      wsh.shared_group = E;
    }
    const bool small = gr.stream_rows > 0;
    if (e == hipSuccess && small)
      e = timed(q4 ? "gateup_q4" : "gateup_fp8", s,
                [&] { return moe::launch_gateup_q_stream(gr, qw, w.x16, T, w.h, shp, H, I, E, true, s); });
    if (e == hipSuccess)
      e = timed(q4 ? "gateup_tile_q4" : "gateup_tile_fp8", s, [&] {
        return moe::launch_gateup_tile_quant(gr, wsh, qw, static_cast<const uint16_t*>(x), w.x16, w.h, H, I, s);
      });
    if (e == hipSuccess && small)
      e = timed(q4 ? "down_q4" : "down_fp8", s,
                [&] { return moe::launch_down_q_stream(gr, qw, w.h, y_rows, shp, H, I, E, true, s); });
    if (e == hipSuccess)
      e = timed(q4 ? "down_tile_q4" : "down_tile_fp8", s,
                [&] { return moe::launch_down_tile_quant(gr, wsh, qw, w.h, y_rows, H, I, s); });
  } else {
    if (e == hipSuccess)
      e = timed(q4 ? "gateup_q4" : "gateup_fp8", s,
                [&] { return moe::launch_gateup_q_stream(gr, qw, w.x16, T, w.h, shp, H, I, E, false, s); });
    if (e == hipSuccess)
      e = timed(q4 ? "down_q4" : "down_fp8", s,
                [&] { return moe::launch_down_q_stream(gr, qw, w.h, y_rows, shp, H, I, E, false, s); });
  }
  if (e != hipSuccess) return device_status(e, "experts");

  e = timed("combine", s, [&] {
    return moe::launch_combine(y_rows, true, w.pair_row, weights, shared ? y_rows + P * H : nullptr, y, true, T, K,
                               H, s);
  });
  return device_status(e, "combine");
}

// ----------------------------------------------------------------------------- no-allocation forward
// Scratch of moe_forward_noalloc: a file-scope device array that every GPU the library runs on holds
// (its own copy, at its own address) until the process ends.  In host code `scratch` names a host
// stand-in, not device memory: host code uses only the per-device address hipGetSymbolAddress gives.
constexpr size_t kNoAllocScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, looked up once per device (with that device
// current) and kept.
int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "moe_forward_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "moe_forward_noalloc: device %d beyond the %d the library tracks", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOE_ERR_DEVICE, "moe_forward_noalloc: hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_workspace_size(const moe_config* cfg, int32_t op, int64_t rows, int32_t n_groups) {
  if (check_config(cfg) != MOE_OK) return 0;
  if (rows < 0) {
    fail(MOE_ERR_INVALID_ARG, "negative rows");
    return 0;
  }
  Carver cv(nullptr);
  switch (op) {
    case MOE_OP_ROUTE:
      cv.take<float>((int64_t)moe::router_nsplit(rows, cfg->hidden_size, cfg->n_routed_experts,
                                                 cfg->dtype == MOE_BF16) * rows * cfg->n_routed_experts);
      break;
    case MOE_OP_PERMUTE:
      cv.take<int32_t>(moe::permute_scratch_ints(rows * cfg->top_k, cfg->n_routed_experts));
      break;
    case MOE_OP_GROUPED_SWIGLU:
      if (n_groups < 1 || n_groups > kMaxGroups) {
        fail(MOE_ERR_INVALID_ARG, "n_groups must be in [1, %d]", kMaxGroups);
        return 0;
      }
      carve_swiglu(cv, cfg, n_groups, rows);
      break;
    case MOE_OP_COMBINE:
      break;
    case MOE_OP_FORWARD:
      if (check_tokens(rows, cfg) != MOE_OK) return 0;
      carve_forward(cv, cfg, rows, true);
      break;
    case MOE_OP_FORWARD_ROUTED:
      if (check_tokens(rows, cfg) != MOE_OK) return 0;
      carve_forward(cv, cfg, rows, false);
      break;
    case MOE_OP_FORWARD_Q4:
    case MOE_OP_FORWARD_FP8:
      if (check_config_quant(cfg, op == MOE_OP_FORWARD_Q4 ? moe::QFormat::kInt4 : moe::QFormat::kFp8) != MOE_OK ||
          check_tokens(rows, cfg) != MOE_OK)
        return 0;
      carve_quant(cv, cfg, rows, op == MOE_OP_FORWARD_Q4 ? moe::QFormat::kInt4 : moe::QFormat::kFp8);
      break;
    default:
      fail(MOE_ERR_INVALID_ARG, "unknown op %d", op);
      return 0;
  }
  ok();
  return cv.used;
}

int moe_route(const moe_config* cfg, int64_t T, const void* x, const void* w_router, const float* score_bias,
              const float* logit_offset, int32_t* topk_ids, float* topk_weights, void* workspace,
              size_t workspace_bytes, void* stream) {
  prof_reset();
  int st = check_config(cfg);
  if (st) return st;
  if ((st = check_tokens(T, cfg))) return st;
  if (T == 0) return ok();
  if (!x || !w_router || !topk_ids || !topk_weights)
    return fail(MOE_ERR_INVALID_ARG, "moe_route: x, w_router, topk_ids and topk_weights are required");
  if ((st = check_aligned("moe_route", {{x, 16, "x"}, {w_router, 16, "w_router"}, {score_bias, 4, "score_bias"},
                                        {logit_offset, 4, "logit_offset"}, {topk_ids, 4, "topk_ids"},
                                        {topk_weights, 4, "topk_weights"}})))
    return st;
  const int H = cfg->hidden_size, E = cfg->n_routed_experts, K = cfg->top_k;
  const bool bf16 = cfg->dtype == MOE_BF16;
  if (bf16 && ((st = check_span("x [T, H]", T * H * 2)) || (st = check_span("w_router [E, H]", (int64_t)E * H * 2))))
    return st;
  Carver cv(workspace);
  const int nsplit = moe::router_nsplit(T, H, E, bf16);
  float* part = cv.take<float>((int64_t)nsplit * T * E);
  if ((st = check_ws(workspace, workspace_bytes, cv.used))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = run_router(cfg, T, x, w_router, part, s);
  if (e != hipSuccess) return device_status(e, "router logits");
  e = timed("topk", s, [&] {
    return moe::launch_topk(part, nsplit, logit_offset, score_bias, T, E, K, cfg->routed_scaling_factor, topk_ids,
                            topk_weights, s);
  });
  return device_status(e, "top-k");
}

int moe_permute(const moe_config* cfg, int64_t T, const int32_t* topk_ids, int32_t* expert_offsets,
                int32_t* row_token, int32_t* pair_row, const void* x, void* x_perm, void* workspace,
                size_t workspace_bytes, void* stream) {
  prof_reset();
  int st = check_config(cfg);
  if (st) return st;
  if ((st = check_tokens(T, cfg))) return st;
  if (T == 0) return ok();
  if (!topk_ids || !expert_offsets || !row_token || !pair_row)
    return fail(MOE_ERR_INVALID_ARG, "moe_permute: topk_ids, expert_offsets, row_token and pair_row are required");
  if ((x == nullptr) != (x_perm == nullptr))
    return fail(MOE_ERR_INVALID_ARG, "moe_permute: x and x_perm must both be given or both be NULL");
  if ((st = check_aligned("moe_permute", {{topk_ids, 4, "topk_ids"}, {expert_offsets, 4, "expert_offsets"},
                                          {row_token, 4, "row_token"}, {pair_row, 4, "pair_row"}, {x, 16, "x"},
                                          {x_perm, 16, "x_perm"}})))
    return st;
  const int E = cfg->n_routed_experts, K = cfg->top_k;
  Carver cv(workspace);
  int32_t* scratch = cv.take<int32_t>(moe::permute_scratch_ints(T * K, E));
  if ((st = check_ws(workspace, workspace_bytes, cv.used))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool fused = moe::permute_plan_fused(T * K, E, 0);
  hipError_t e = timed("permute", s, [&] {
    return fused ? moe::launch_permute_plan(topk_ids, T, K, E, expert_offsets, row_token, pair_row, false,
                                            moe::Groups{}, nullptr, nullptr, cfg->hidden_size, s)
                 : moe::launch_permute(topk_ids, T, K, E, expert_offsets, row_token, pair_row, scratch, false, s);
  });
  if (e != hipSuccess) return device_status(e, "permute");
  if (x) {
    e = timed("gather", s, [&] {
      return moe::launch_gather_rows(x, row_token, x_perm, T * K, cfg->hidden_size, (int)elem_bytes(cfg->dtype), s);
    });
    if (e != hipSuccess) return device_status(e, "gather");
  }
  return ok();
}

int moe_grouped_swiglu(const moe_config* cfg, int32_t n_groups, const int32_t* group_offsets, int64_t max_rows,
                       const void* x, const int32_t* row_index, const void* w_gate, const void* w_up,
                       const void* w_down, const float* row_scale, void* y_rows, int32_t y_dtype, void* workspace,
                       size_t workspace_bytes, void* stream) {
  prof_reset();
  int st = check_config(cfg);
  if (st) return st;
  if (n_groups < 1 || n_groups > kMaxGroups) return fail(MOE_ERR_INVALID_ARG, "n_groups must be in [1, %d]", kMaxGroups);
  if (max_rows < 0) return fail(MOE_ERR_INVALID_ARG, "negative max_rows");
  if (max_rows > 0x7fffffffLL) return fail(MOE_ERR_UNSUPPORTED, "max_rows exceeds 2^31-1");
  if (max_rows == 0) return ok();
  if (!group_offsets || !x || !w_gate || !w_up || !w_down || !y_rows)
    return fail(MOE_ERR_INVALID_ARG, "moe_grouped_swiglu: group_offsets, x, weights and y_rows are required");
  if (y_dtype != MOE_F32 && y_dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "y_dtype %d", y_dtype);
  if ((st = check_aligned("moe_grouped_swiglu", {{group_offsets, 4, "group_offsets"}, {x, 16, "x"},
                                                 {row_index, 4, "row_index"}, {w_gate, 16, "w_gate"},
                                                 {w_up, 16, "w_up"}, {w_down, 16, "w_down"},
                                                 {row_scale, 4, "row_scale"}, {y_rows, 16, "y_rows"}})))
    return st;
  if (cfg->dtype == MOE_F32 && y_dtype != MOE_F32)
    return fail(MOE_ERR_UNSUPPORTED, "fp32 layers produce fp32 y_rows");
  if (cfg->dtype == MOE_BF16) {
    const int64_t H = cfg->hidden_size, I = cfg->moe_intermediate_size;
    if ((!row_index && (st = check_span("x [max_rows, H]", max_rows * H * 2))) ||
        (st = check_span("h [max_rows, I]", max_rows * I * 2)) || (st = check_span("an expert weight [I, H]", I * H * 2)))
      return st;
  }
  Carver cv(workspace);
  SwigluWs w = carve_swiglu(cv, cfg, n_groups, max_rows);
  if ((st = check_ws(workspace, workspace_bytes, cv.used))) return st;
  w.g.group_offsets = group_offsets;
  w.g.row_index = row_index;
  moe::Weights wt;
  wt.gate = w_gate;
  wt.up = w_up;
  wt.down = w_down;
  hipError_t e = run_swiglu(cfg, w.g, wt, x, w.h, w.part, row_scale, y_rows, y_dtype == MOE_BF16,
                            static_cast<hipStream_t>(stream));
  return device_status(e, "grouped swiglu");
}

int moe_combine(const moe_config* cfg, int64_t T, const void* y_rows, int32_t y_dtype, const int32_t* pair_row,
                const float* topk_weights, const void* y_shared, void* y, void* stream) {
  prof_reset();
  int st = check_config(cfg);
  if (st) return st;
  if ((st = check_tokens(T, cfg))) return st;
  if (T == 0) return ok();
  if (!y_rows || !pair_row || !topk_weights || !y)
    return fail(MOE_ERR_INVALID_ARG, "moe_combine: y_rows, pair_row, topk_weights and y are required");
  if ((st = check_aligned("moe_combine", {{y_rows, 16, "y_rows"}, {pair_row, 4, "pair_row"},
                                          {topk_weights, 4, "topk_weights"}, {y_shared, 16, "y_shared"},
                                          {y, 16, "y"}})))
    return st;
  if (y_dtype != MOE_F32 && y_dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "y_dtype %d", y_dtype);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = timed("combine", s, [&] {
    return moe::launch_combine(y_rows, y_dtype == MOE_BF16, pair_row, topk_weights, y_shared, y,
                               cfg->dtype == MOE_BF16, T, cfg->top_k, cfg->hidden_size, s);
  });
  return device_status(e, "combine");
}

int moe_forward(const moe_config* cfg, int64_t T, const void* x, const void* w_router, const float* score_bias,
                const float* logit_offset, const void* w_gate, const void* w_up, const void* w_down,
                const void* ws_gate, const void* ws_up, const void* ws_down, void* y, int32_t* topk_ids_out,
                float* topk_weights_out, void* workspace, size_t workspace_bytes, void* stream) {
  prof_reset();
  int st = check_config(cfg);
  if (st) return st;
  if ((st = check_tokens(T, cfg))) return st;
  if (T == 0) return ok();
  if (!x || !w_router || !w_gate || !w_up || !w_down || !y)
    return fail(MOE_ERR_INVALID_ARG, "moe_forward: x, w_router, expert weights and y are required");
  if (cfg->n_shared_experts == 1 && (!ws_gate || !ws_up || !ws_down))
    return fail(MOE_ERR_INVALID_ARG, "moe_forward: shared expert weights are required");
  if ((st = check_aligned("moe_forward", {{x, 16, "x"}, {w_router, 16, "w_router"}, {w_gate, 16, "w_gate"},
                                          {w_up, 16, "w_up"}, {w_down, 16, "w_down"}, {ws_gate, 16, "ws_gate"},
                                          {ws_up, 16, "ws_up"}, {ws_down, 16, "ws_down"}, {y, 16, "y"},
                                          {score_bias, 4, "score_bias"}, {logit_offset, 4, "logit_offset"},
                                          {topk_ids_out, 4, "topk_ids_out"},
                                          {topk_weights_out, 4, "topk_weights_out"}})))
    return st;
  if ((st = check_forward_spans(cfg, T))) return st;
  const int H = cfg->hidden_size, E = cfg->n_routed_experts, K = cfg->top_k;
  const bool bf16 = cfg->dtype == MOE_BF16;
  Carver cv(workspace);
  ForwardWs w = carve_forward(cv, cfg, T, true);
  if ((st = check_ws(workspace, workspace_bytes, cv.used))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* ids = topk_ids_out ? topk_ids_out : w.ids;
  float* weights = topk_weights_out ? topk_weights_out : w.weights;
  hipError_t e = run_router(cfg, T, x, w_router, w.router_part, s);
  if (e != hipSuccess) return device_status(e, "router logits");
  e = timed("topk", s, [&] {
    return moe::launch_topk(w.router_part, moe::router_nsplit(T, H, E, bf16), logit_offset, score_bias, T, E, K,
                            cfg->routed_scaling_factor, ids, weights, s);
  });
  if (e != hipSuccess) return device_status(e, "top-k");
  return run_after_routing(cfg, T, x, ids, weights, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, y, w, s);
}

int moe_forward_noalloc(const moe_config* cfg, int64_t T, const void* x, const void* w_router,
                        const float* score_bias, const float* logit_offset, const void* w_gate, const void* w_up,
                        const void* w_down, const void* ws_gate, const void* ws_up, const void* ws_down, void* y,
                        int32_t* topk_ids_out, float* topk_weights_out, void* stream) {
  prof_reset();
  int st = check_config(cfg);
  if (st) return st;
  if ((st = check_tokens(T, cfg))) return st;
  if (T == 0) return ok();
  Carver cv(nullptr);
  carve_forward(cv, cfg, T, true);
  if (cv.used > kNoAllocScratchBytes)
    return fail(MOE_ERR_WORKSPACE,
                "moe_forward_noalloc: T=%lld needs %zu bytes of scratch, above its fixed %zu bytes "
                "(use moe_forward with a workspace)",
                (long long)T, cv.used, kNoAllocScratchBytes);
  void* ws = nullptr;
  if ((st = scratch_of_current_device(&ws))) return st;
  return moe_forward(cfg, T, x, w_router, score_bias, logit_offset, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, y,
                     topk_ids_out, topk_weights_out, ws, kNoAllocScratchBytes, stream);
}

int moe_forward_routed(const moe_config* cfg, int64_t T, const void* x, const int32_t* topk_ids,
                       const float* topk_weights, const void* w_gate, const void* w_up, const void* w_down,
                       const void* ws_gate, const void* ws_up, const void* ws_down, void* y, void* workspace,
                       size_t workspace_bytes, void* stream) {
  prof_reset();
  int st = check_config(cfg);
  if (st) return st;
  if ((st = check_tokens(T, cfg))) return st;
  if (T == 0) return ok();
  if (!x || !topk_ids || !topk_weights || !w_gate || !w_up || !w_down || !y)
    return fail(MOE_ERR_INVALID_ARG, "moe_forward_routed: x, routing, expert weights and y are required");
  if (cfg->n_shared_experts == 1 && (!ws_gate || !ws_up || !ws_down))
    return fail(MOE_ERR_INVALID_ARG, "moe_forward_routed: shared expert weights are required");
  if ((st = check_aligned("moe_forward_routed", {{x, 16, "x"}, {topk_ids, 4, "topk_ids"},
                                                 {topk_weights, 4, "topk_weights"}, {w_gate, 16, "w_gate"},
                                                 {w_up, 16, "w_up"}, {w_down, 16, "w_down"},
                                                 {ws_gate, 16, "ws_gate"}, {ws_up, 16, "ws_up"},
                                                 {ws_down, 16, "ws_down"}, {y, 16, "y"}})))
    return st;
  if ((st = check_forward_spans(cfg, T))) return st;
  Carver cv(workspace);
  ForwardWs w = carve_forward(cv, cfg, T, false);
  if ((st = check_ws(workspace, workspace_bytes, cv.used))) return st;
  return run_after_routing(cfg, T, x, topk_ids, topk_weights, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, y, w,
                           static_cast<hipStream_t>(stream));
}

int moe_forward_q4(const moe_config* cfg, int64_t T, const void* x, const void* w_router, const float* score_bias,
                   const float* logit_offset, const uint32_t* gate_codes, const uint16_t* gate_scales,
                   const uint32_t* up_codes, const uint16_t* up_scales, const uint32_t* down_codes,
                   const uint16_t* down_scales, const void* ws_gate, const void* ws_up, const void* ws_down, void* y,
                   int32_t* topk_ids_out, float* topk_weights_out, void* workspace, size_t workspace_bytes,
                   void* stream) {
  const moe::QWeights qw{moe::QFormat::kInt4, gate_codes, gate_scales, up_codes, up_scales, down_codes, down_scales};
  return forward_quant("moe_forward_q4", cfg, T, x, w_router, score_bias, logit_offset, qw, ws_gate, ws_up, ws_down,
                       y, topk_ids_out, topk_weights_out, workspace, workspace_bytes, stream);
}

int moe_forward_fp8(const moe_config* cfg, int64_t T, const void* x, const void* w_router, const float* score_bias,
                    const float* logit_offset, const uint8_t* gate_codes, const float* gate_scales,
                    const uint8_t* up_codes, const float* up_scales, const uint8_t* down_codes,
                    const float* down_scales, const void* ws_gate, const void* ws_up, const void* ws_down, void* y,
                    int32_t* topk_ids_out, float* topk_weights_out, void* workspace, size_t workspace_bytes,
                    void* stream) {
  const moe::QWeights qw{moe::QFormat::kFp8, gate_codes, gate_scales, up_codes, up_scales, down_codes, down_scales};
  return forward_quant("moe_forward_fp8", cfg, T, x, w_router, score_bias, logit_offset, qw, ws_gate, ws_up, ws_down,
                       y, topk_ids_out, topk_weights_out, workspace, workspace_bytes, stream);
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

int moe_profile_events(void* const* events, int32_t n_events) {
  if (n_events < 0 || (n_events > 0 && events == nullptr))
    return fail(MOE_ERR_INVALID_ARG, "moe_profile_events: need events for n_events > 0");
  g_prof.events = n_events > 0 ? events : nullptr;
  g_prof.n_events = n_events;
  g_prof.count = 0;
  return ok();
}

int32_t moe_profile_count(void) { return g_prof.count; }

const char* moe_profile_kernel(int32_t i) {
  return (i >= 0 && i < g_prof.count && i < kMaxProfiled && g_prof.names[i]) ? g_prof.names[i] : "";
}

}  // extern "C"
