// libmoe C ABI: argument validation, workspace carving and launch order.
// The operations themselves are described where they are declared
// (include/moe.h) and implemented in the kernels' files.
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "../../include/moe.h"
#include "launch.h"

namespace moe {
// dispatch.hip: T = 0, counts [E] and offsets [E + 1] (either may be null)
// set to zero
hipError_t launch_dispatch_empty(const moe_cfg& c, int32_t* counts, int32_t* offsets,
                                 hipStream_t s);
}  // namespace moe

namespace {

thread_local int g_last_hip_error = 0;
// polls of a split part's ready flag before its consumer gives up
// (moe_set_split_wait)
std::atomic<int> g_split_wait{moe::kSplitWaitDefault};

constexpr int kMaxE = 1024;
constexpr int kMaxK = 16;
constexpr size_t kAlign = 256;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool dev_ok(const void* p) { return p != nullptr && aligned16(p); }
bool opt_ok(const void* p) { return p == nullptr || aligned16(p); }

size_t act_size(const moe_cfg& c) { return c.act_dtype == MOE_BF16 ? 2 : 4; }
bool is_a8(const moe_cfg& c) { return c.w_dtype == MOE_MXFP4_A8; }
bool is_mx(const moe_cfg& c) { return c.w_dtype == MOE_MXFP4 || is_a8(c); }

int check_cfg(const moe_cfg* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->T < 0 || c->D < 8 || c->E < 1 || c->F < 8 || c->top_k < 1) return MOE_ERR_INVALID_ARG;
  if (c->D % 8 || c->F % 8) return MOE_ERR_INVALID_ARG;
  if (c->top_k > c->E) return MOE_ERR_INVALID_ARG;
  if (c->gating < MOE_GATE_SOFTMAX || c->gating > MOE_GATE_SQRT_SOFTPLUS) return MOE_ERR_INVALID_ARG;
  if (c->renorm != 0 && c->renorm != 1) return MOE_ERR_INVALID_ARG;
  if (isnan(c->clamp) || isinf(c->clamp)) return MOE_ERR_INVALID_ARG;
  if (c->shared_F < 0) return MOE_ERR_INVALID_ARG;
  const bool f32 = c->act_dtype == MOE_F32 && c->w_dtype == MOE_F32;
  const bool bf = c->act_dtype == MOE_BF16 &&
                  (c->w_dtype == MOE_BF16 || c->w_dtype == MOE_MXFP4 || c->w_dtype == MOE_MXFP4_A8);
  if (!f32 && !bf) return MOE_ERR_INVALID_ARG;
  if (c->E > kMaxE || c->top_k > kMaxK) return MOE_ERR_UNSUPPORTED;
  // row and element indices are int32 on the device side
  if ((long long)c->T * c->top_k > 0x7FFFFFFFLL) return MOE_ERR_UNSUPPORTED;
  if (bf) {
    if (c->D % 32 || c->F % 32) return MOE_ERR_UNSUPPORTED;  // GEMM K steps of 32
    if (is_a8(*c) && (c->D % 64 || c->F % 64)) return MOE_ERR_UNSUPPORTED;  // and of 64
  }
  if (c->shared_F > 0) {
    if (c->act_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (c->shared_F % 32) return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

int check_weights(const moe_cfg& c, const moe_weights* w) {
  if (!w) return MOE_ERR_INVALID_ARG;
  if (!dev_ok(w->W_gate) || !dev_ok(w->W_up) || !dev_ok(w->W_down)) return MOE_ERR_INVALID_ARG;
  if (is_mx(c)) {
    if (!dev_ok(w->S_gate) || !dev_ok(w->S_up) || !dev_ok(w->S_down)) return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

int check_shared(const moe_cfg& c, const moe_weights* w) {
  if (c.shared_F == 0) return MOE_OK;
  if (!w || !dev_ok(w->Ws_gate) || !dev_ok(w->Ws_up) || !dev_ok(w->Ws_down))
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip_error = static_cast<int>(e);
  return MOE_ERR_HIP;
}

// Sequential carving of a caller-provided workspace.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* p) : base(static_cast<char*>(p)) {}
  void* take(size_t bytes) {
    off = moe::align_up(off, kAlign);
    void* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  }
};

size_t dispatch_ws(const moe_cfg& c) {
  return moe::align_up((size_t)c.E * moe::num_chunks(c) * 4, kAlign);
}
// MXFP8 copy of `rows` activation rows of width K: codes, then the scales
// in the grouped layout the GEMM reads ([ceil(K/512)][rows][16])
size_t mxfp8_bytes(size_t rows, int K) {
  return moe::align_up(rows * K, kAlign) + moe::align_up((size_t)((K + 511) / 512) * rows * 16, kAlign);
}
// expert FFN workspace: the tile map, then (bf16 activations) the split
// flags and partial-sum slots of the grouped GEMMs, then (MXFP8 activations)
// the MXFP8 copy of x that a gathered gate/up launch reads
size_t tilemap_bytes(const moe_cfg& c) { return moe::align_up(moe::tilemap_ints(c) * 4, kAlign); }
size_t xq_bytes(const moe_cfg& c) { return is_a8(c) ? mxfp8_bytes(c.T, c.D) : 0; }
size_t ffn_ws(const moe_cfg& c) { return tilemap_bytes(c) + moe::split_bytes(c) + xq_bytes(c); }
int32_t* split_flags_of(const moe_cfg& c, int32_t* tilemap) {
  if (!moe::gemm_splits(c)) return nullptr;
  return reinterpret_cast<int32_t*>(reinterpret_cast<char*>(tilemap) + tilemap_bytes(c));
}
float* split_ws_of(const moe_cfg& c, int32_t* tilemap) {
  if (!moe::gemm_splits(c)) return nullptr;
  return reinterpret_cast<float*>(reinterpret_cast<char*>(split_flags_of(c, tilemap)) +
                                  moe::kSplitFlagBytes);
}
uint8_t* xq_of(const moe_cfg& c, int32_t* tilemap) {
  if (!is_a8(c)) return nullptr;
  return reinterpret_cast<uint8_t*>(tilemap) + tilemap_bytes(c) + moe::split_bytes(c);
}

size_t route_ws(const moe_cfg& c) {
  return moe::router_screen_applies(c) ? moe::router_screen_ws_bytes(c) : 0;
}

struct ForwardWs {
  void* route;  // screened router's workspace (when it applies)
  int32_t *idx, *counts, *offsets, *slot_pos, *perm, *chunk_ws, *tilemap;
  float *w, *y_perm, *y_shared;
  void *x_perm, *H, *H_shared;
  size_t bytes;
};

ForwardWs carve_forward(const moe_cfg& c, void* ws) {
  Carver cv(ws);
  ForwardWs f;
  const size_t tk = (size_t)c.T * c.top_k;
  f.idx = static_cast<int32_t*>(cv.take(tk * 4));
  f.w = static_cast<float*>(cv.take(tk * 4));
  f.counts = static_cast<int32_t*>(cv.take((size_t)c.E * 4));
  f.offsets = static_cast<int32_t*>(cv.take(((size_t)c.E + 1) * 4));
  f.slot_pos = static_cast<int32_t*>(cv.take(tk * 4));
  f.perm = static_cast<int32_t*>(cv.take(tk * 4));
  f.chunk_ws = static_cast<int32_t*>(cv.take(dispatch_ws(c)));
  f.route = route_ws(c) ? cv.take(route_ws(c)) : nullptr;
  f.tilemap = static_cast<int32_t*>(cv.take(ffn_ws(c)));
  // bf16: gate/up gathers its rows from x through perm (no dispatched copy)
  f.x_perm = c.act_dtype == MOE_F32 ? cv.take(tk * c.D * act_size(c)) : nullptr;
  f.H = cv.take(tk * c.F * act_size(c));
  f.y_perm = static_cast<float*>(cv.take(tk * c.D * 4));
  f.H_shared = c.shared_F > 0 ? cv.take((size_t)c.T * c.shared_F * 2) : nullptr;
  f.y_shared = c.shared_F > 0 ? static_cast<float*>(cv.take((size_t)c.T * c.D * 4)) : nullptr;
  f.bytes = moe::align_up(cv.off, kAlign);
  return f;
}

// MXFP4 weights (with bf16 or MXFP8 activations) run an expert's last
// M-tile of at most 128 rows as a wide tile; bf16 weights do not.
bool wide_tiles(const moe_cfg& c) { return is_mx(c); }

moe::GemmProblem routed_problem(const moe_cfg& c, const int32_t* offsets, int32_t* tilemap) {
  moe::GemmProblem g{};
  g.tilemap = tilemap;
  g.offsets = offsets;
  g.rows = c.T * c.top_k;
  g.max_tiles = moe::max_mtiles(c);
  g.E = c.E;
  g.mxfp4 = is_mx(c);
  g.clamp = c.clamp;
  g.split_flags = split_flags_of(c, tilemap);
  g.split_ws = split_ws_of(c, tilemap);
  g.split_wait = g_split_wait.load(std::memory_order_relaxed);
  return g;
}

// gate + up with the SwiGLU epilogue -> H
// (gather: nullptr, x_perm holds the dispatched rows; else x_perm is x and
// routed row r reads row gather[r] of it). With MXFP8 activations H is
// written as MXFP8 (codes [T*k][F], then grouped scales); the dispatched
// x_perm is MXFP8 already (codes [T*k][D], then grouped scales), and x
// (gathered) is first quantised into the workspace's MXFP8 copy of x.
hipError_t run_gate_up(const moe_cfg& c, const void* x_perm, const int32_t* gather,
                       const int32_t* offsets, const moe_weights& w, void* H, int32_t* tilemap,
                       hipStream_t s) {
  if (c.act_dtype == MOE_F32)
    return moe::launch_ffn_f32_gate_up(c, static_cast<const float*>(x_perm), offsets,
                                       static_cast<const float*>(w.W_gate),
                                       static_cast<const float*>(w.W_up), static_cast<float*>(H), s);
  hipError_t e = moe::launch_tilemap(c, offsets, tilemap, split_flags_of(c, tilemap), wide_tiles(c), s);
  if (e != hipSuccess) return e;
  moe::GemmProblem g = routed_problem(c, offsets, tilemap);
  g.A = x_perm;
  g.gather = gather;
  g.gather_rows = c.T;
  g.K = c.D;
  g.N = c.F;
  g.B0 = w.W_gate;
  g.B1 = w.W_up;
  g.S0 = w.S_gate;
  g.S1 = w.S_up;
  g.out = H;
  if (!is_a8(c)) return moe::launch_gemm_swiglu(g, s);
  if (gather) {
    uint8_t* xq = xq_of(c, tilemap);
    uint8_t* xs = xq + moe::align_up((size_t)c.T * c.D, kAlign);
    e = moe::launch_quant_mxfp8(x_perm, c.T, c.D, xq, xs, true, s);
    if (e != hipSuccess) return e;
    g.A = xq;
    g.SA = xs;
  } else {
    g.SA = static_cast<const uint8_t*>(x_perm) + (size_t)g.rows * c.D;  // scales after codes
  }
  return moe::launch_gemm_a8(g, true, s);
}

// down projection -> y_perm; rebuild_map = false reuses the tile map that a
// preceding run_gate_up left in the same workspace
hipError_t run_down(const moe_cfg& c, const void* H, const int32_t* offsets, const moe_weights& w,
                    float* y_perm, int32_t* tilemap, bool rebuild_map, hipStream_t s) {
  if (c.act_dtype == MOE_F32)
    return moe::launch_ffn_f32_down(c, static_cast<const float*>(H), offsets,
                                    static_cast<const float*>(w.W_down), y_perm, s);
  if (rebuild_map) {
    hipError_t e = moe::launch_tilemap(c, offsets, tilemap, split_flags_of(c, tilemap), wide_tiles(c), s);
    if (e != hipSuccess) return e;
  }
  moe::GemmProblem g = routed_problem(c, offsets, tilemap);
  if (g.split_flags) g.split_flags += moe::kSplitSlots;  // the down launch's flag bank
  g.A = H;
  g.K = c.F;
  g.N = c.D;
  g.B0 = w.W_down;
  g.S0 = w.S_down;
  g.out = y_perm;
  if (!is_a8(c)) return moe::launch_gemm_down(g, s);
  g.SA = static_cast<const uint8_t*>(H) + (size_t)g.rows * c.F;  // MXFP8 H: grouped scales after codes
  return moe::launch_gemm_a8(g, false, s);
}

hipError_t run_expert_ffn(const moe_cfg& c, const void* x_perm, const int32_t* gather,
                          const int32_t* offsets, const moe_weights& w, void* H, float* y_perm,
                          int32_t* tilemap, hipStream_t s) {
  hipError_t e = run_gate_up(c, x_perm, gather, offsets, w, H, tilemap, s);
  if (e != hipSuccess) return e;
  return run_down(c, H, offsets, w, y_perm, tilemap, false, s);
}

hipError_t run_shared(const moe_cfg& c, const void* x, const moe_weights& w, void* H_shared,
                      float* y_shared, hipStream_t s) {
  moe::GemmProblem g{};
  g.tilemap = nullptr;
  g.offsets = nullptr;
  g.rows = c.T;
  g.max_tiles = moe::ceil_div(c.T, moe::kBM);
  g.E = 1;
  g.mxfp4 = 0;
  g.clamp = c.clamp;
  g.A = x;
  g.K = c.D;
  g.N = c.shared_F;
  g.B0 = w.Ws_gate;
  g.B1 = w.Ws_up;
  g.out = H_shared;
  hipError_t e = moe::launch_gemm_swiglu(g, s);
  if (e != hipSuccess) return e;
  g.A = H_shared;
  g.K = c.shared_F;
  g.N = c.D;
  g.B0 = w.Ws_down;
  g.B1 = nullptr;
  g.out = y_shared;
  return moe::launch_gemm_down(g, s);
}

}  // namespace

extern "C" {

int moe_version(void) { return MOE_ABI_VERSION; }

int moe_set_split_wait(int polls) {
  if (polls < 0) return MOE_ERR_INVALID_ARG;
  return g_split_wait.exchange(polls);
}

int moe_last_hip_error(void) { return g_last_hip_error; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    case MOE_ERR_SCRATCH: return "beyond the fixed scratch of the no-allocation entry point";
    default: return "unknown status";
  }
}

int moe_workspace_size(const moe_cfg* cfg, int kind, size_t* bytes) {
  int st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  switch (kind) {
    case MOE_WS_DISPATCH: *bytes = dispatch_ws(*cfg); return MOE_OK;
    case MOE_WS_EXPERT_FFN: *bytes = cfg->act_dtype == MOE_F32 ? 0 : ffn_ws(*cfg); return MOE_OK;
    case MOE_WS_FORWARD: *bytes = carve_forward(*cfg, nullptr).bytes; return MOE_OK;
    case MOE_WS_ROUTE: *bytes = route_ws(*cfg); return MOE_OK;
    default: return MOE_ERR_INVALID_ARG;
  }
}

int moe_route(const moe_cfg* cfg, const void* x, const float* W_r, const float* bias,
              int32_t* topk_idx, float* topk_w, float* logits, void* stream) {
  int st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (!dev_ok(x) || !dev_ok(W_r) || !dev_ok(topk_idx) || !dev_ok(topk_w) || !opt_ok(bias) ||
      !opt_ok(logits))
    return MOE_ERR_INVALID_ARG;
  if (cfg->T == 0) return MOE_OK;
  return hip_status(moe::launch_router(*cfg, x, W_r, bias, topk_idx, topk_w, logits,
                                       static_cast<hipStream_t>(stream)));
}

int moe_route_screened(const moe_cfg* cfg, const void* x, const float* W_r, const float* bias,
                       int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes, void* stream) {
  int st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (!dev_ok(x) || !dev_ok(W_r) || !dev_ok(topk_idx) || !dev_ok(topk_w) || !opt_ok(bias))
    return MOE_ERR_INVALID_ARG;
  const size_t need = route_ws(*cfg);
  if (need && (!ws || !aligned16(ws) || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  if (cfg->T == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!need) return hip_status(moe::launch_router(*cfg, x, W_r, bias, topk_idx, topk_w, nullptr, s));
  return hip_status(moe::launch_router_screened(*cfg, x, W_r, bias, topk_idx, topk_w, ws, s));
}

int moe_dispatch(const moe_cfg* cfg, const int32_t* topk_idx, const void* x, int32_t* counts,
                 int32_t* offsets, int32_t* slot_pos, int32_t* perm_token, void* x_perm,
                 void* ws, size_t ws_bytes, void* stream) {
  int st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (!dev_ok(topk_idx) || !dev_ok(x) || !dev_ok(counts) || !dev_ok(offsets) ||
      !dev_ok(slot_pos) || !dev_ok(perm_token) || !opt_ok(x_perm))
    return MOE_ERR_INVALID_ARG;
  if (!ws || !aligned16(ws) || ws_bytes < dispatch_ws(*cfg)) return MOE_ERR_WORKSPACE;
  if (cfg->T == 0)
    return hip_status(moe::launch_dispatch_empty(*cfg, counts, offsets,
                                                 static_cast<hipStream_t>(stream)));
  return hip_status(moe::launch_dispatch(*cfg, topk_idx, x, counts, offsets, slot_pos, perm_token,
                                         x_perm, static_cast<int32_t*>(ws),
                                         static_cast<hipStream_t>(stream)));
}

int moe_dispatch_noalloc(const moe_cfg* cfg, const int32_t* topk_idx, const void* x,
                         int32_t* counts, int32_t* offsets, int32_t* slot_pos,
                         int32_t* perm_token, void* x_perm, void* stream) {
  int st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (!dev_ok(topk_idx) || !dev_ok(x) || !dev_ok(counts) || !dev_ok(offsets) ||
      !dev_ok(slot_pos) || !dev_ok(perm_token) || !opt_ok(x_perm))
    return MOE_ERR_INVALID_ARG;
  if ((size_t)cfg->E * moe::num_chunks(*cfg) > moe::kDispatchScratchInts)
    return MOE_ERR_SCRATCH;
  if (cfg->T == 0)
    return hip_status(moe::launch_dispatch_empty(*cfg, counts, offsets,
                                                 static_cast<hipStream_t>(stream)));
  int32_t* scratch = nullptr;
  hipError_t e = moe::dispatch_scratch(&scratch);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(moe::launch_dispatch(*cfg, topk_idx, x, counts, offsets, slot_pos, perm_token,
                                         x_perm, scratch, static_cast<hipStream_t>(stream)));
}

int moe_expert_ffn(const moe_cfg* cfg, const void* x_perm, const int32_t* offsets,
                   const moe_weights* w, void* H, float* y_perm, void* ws, size_t ws_bytes,
                   void* stream) {
  int st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_weights(*cfg, w)) != MOE_OK) return st;
  if (!dev_ok(x_perm) || !dev_ok(offsets) || !dev_ok(H) || !dev_ok(y_perm))
    return MOE_ERR_INVALID_ARG;
  if (cfg->act_dtype != MOE_F32 && (!ws || !aligned16(ws) || ws_bytes < ffn_ws(*cfg)))
    return MOE_ERR_WORKSPACE;
  if (cfg->T == 0) return MOE_OK;
  return hip_status(run_expert_ffn(*cfg, x_perm, nullptr, offsets, *w, H, y_perm,
                                   static_cast<int32_t*>(ws), static_cast<hipStream_t>(stream)));
}

int moe_expert_gate_up(const moe_cfg* cfg, const void* x_perm, const int32_t* offsets,
                       const moe_weights* w, void* H, void* ws, size_t ws_bytes, void* stream) {
  int st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_weights(*cfg, w)) != MOE_OK) return st;
  if (!dev_ok(x_perm) || !dev_ok(offsets) || !dev_ok(H)) return MOE_ERR_INVALID_ARG;
  if (cfg->act_dtype != MOE_F32 && (!ws || !aligned16(ws) || ws_bytes < ffn_ws(*cfg)))
    return MOE_ERR_WORKSPACE;
  if (cfg->T == 0) return MOE_OK;
  return hip_status(run_gate_up(*cfg, x_perm, nullptr, offsets, *w, H, static_cast<int32_t*>(ws),
                                static_cast<hipStream_t>(stream)));
}

int moe_expert_gate_up_gathered(const moe_cfg* cfg, const void* x, const int32_t* perm_token,
                                const int32_t* offsets, const moe_weights* w, void* H, void* ws,
                                size_t ws_bytes, void* stream) {
  int st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_weights(*cfg, w)) != MOE_OK) return st;
  if (cfg->act_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (!dev_ok(x) || !dev_ok(perm_token) || !dev_ok(offsets) || !dev_ok(H))
    return MOE_ERR_INVALID_ARG;
  if (!ws || !aligned16(ws) || ws_bytes < ffn_ws(*cfg)) return MOE_ERR_WORKSPACE;
  if (cfg->T == 0) return MOE_OK;
  return hip_status(run_gate_up(*cfg, x, perm_token, offsets, *w, H, static_cast<int32_t*>(ws),
                                static_cast<hipStream_t>(stream)));
}

int moe_expert_down(const moe_cfg* cfg, const void* H, const int32_t* offsets,
                    const moe_weights* w, float* y_perm, void* ws, size_t ws_bytes, void* stream) {
  int st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_weights(*cfg, w)) != MOE_OK) return st;
  if (!dev_ok(H) || !dev_ok(offsets) || !dev_ok(y_perm)) return MOE_ERR_INVALID_ARG;
  if (cfg->act_dtype != MOE_F32 && (!ws || !aligned16(ws) || ws_bytes < ffn_ws(*cfg)))
    return MOE_ERR_WORKSPACE;
  if (cfg->T == 0) return MOE_OK;
  return hip_status(run_down(*cfg, H, offsets, *w, y_perm, static_cast<int32_t*>(ws), true,
                             static_cast<hipStream_t>(stream)));
}

int moe_shared_expert(const moe_cfg* cfg, const void* x, const moe_weights* w, void* H_shared,
                      float* y_shared, void* stream) {
  int st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (cfg->shared_F == 0) return MOE_ERR_INVALID_ARG;
  if ((st = check_shared(*cfg, w)) != MOE_OK) return st;
  if (!dev_ok(x) || !dev_ok(H_shared) || !dev_ok(y_shared)) return MOE_ERR_INVALID_ARG;
  if (cfg->T == 0) return MOE_OK;
  return hip_status(run_shared(*cfg, x, *w, H_shared, y_shared, static_cast<hipStream_t>(stream)));
}

int moe_combine(const moe_cfg* cfg, const float* y_perm, const int32_t* slot_pos,
                const float* topk_w, const float* y_shared, void* y, void* stream) {
  int st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (!dev_ok(y_perm) || !dev_ok(slot_pos) || !dev_ok(topk_w) || !opt_ok(y_shared) || !dev_ok(y))
    return MOE_ERR_INVALID_ARG;
  if (cfg->T == 0) return MOE_OK;
  return hip_status(moe::launch_combine(*cfg, y_perm, slot_pos, topk_w, y_shared, y,
                                        static_cast<hipStream_t>(stream)));
}

int moe_quantize_mxfp8(const void* x, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales,
                       void* stream) {
  if (rows < 0 || K <= 0 || K % 32) return MOE_ERR_INVALID_ARG;
  if (!dev_ok(x) || !dev_ok(codes) || !dev_ok(scales)) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  return hip_status(moe::launch_quant_mxfp8(x, rows, K, codes, scales, false,
                                            static_cast<hipStream_t>(stream)));
}

int moe_forward(const moe_cfg* cfg, const void* x, const float* W_r, const float* bias,
                const moe_weights* w, void* y, int32_t* topk_idx, float* topk_w, int32_t* counts,
                int32_t* offsets, void* ws, size_t ws_bytes, void* stream) {
  int st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_weights(*cfg, w)) != MOE_OK) return st;
  if ((st = check_shared(*cfg, w)) != MOE_OK) return st;
  if (!dev_ok(x) || !dev_ok(W_r) || !opt_ok(bias) || !dev_ok(y) || !opt_ok(topk_idx) ||
      !opt_ok(topk_w) || !opt_ok(counts) || !opt_ok(offsets))
    return MOE_ERR_INVALID_ARG;
  const ForwardWs f0 = carve_forward(*cfg, nullptr);
  if (!ws || !aligned16(ws) || ws_bytes < f0.bytes) return MOE_ERR_WORKSPACE;
  if (cfg->T == 0)  // y has no rows; the optional counts and offsets are zero
    return hip_status(moe::launch_dispatch_empty(*cfg, counts, offsets,
                                                 static_cast<hipStream_t>(stream)));
  const moe_cfg& c = *cfg;
  const ForwardWs f = carve_forward(c, ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* idx = topk_idx ? topk_idx : f.idx;
  float* tw = topk_w ? topk_w : f.w;
  int32_t* cnt = counts ? counts : f.counts;
  int32_t* off = offsets ? offsets : f.offsets;
  hipError_t e = f.route ? moe::launch_router_screened(c, x, W_r, bias, idx, tw, f.route, s)
                         : moe::launch_router(c, x, W_r, bias, idx, tw, nullptr, s);
  if (e == hipSuccess)
    e = moe::launch_dispatch(c, idx, x, cnt, off, f.slot_pos, f.perm, f.x_perm, f.chunk_ws, s);
  if (e == hipSuccess) {
    if (f.x_perm)  // fp32 activations: the VALU path reads dispatched rows
      e = run_expert_ffn(c, f.x_perm, nullptr, off, *w, f.H, f.y_perm, f.tilemap, s);
    else
      e = run_expert_ffn(c, x, f.perm, off, *w, f.H, f.y_perm, f.tilemap, s);
  }
  if (e == hipSuccess && c.shared_F > 0) e = run_shared(c, x, *w, f.H_shared, f.y_shared, s);
  if (e == hipSuccess) e = moe::launch_combine(c, f.y_perm, f.slot_pos, tw, f.y_shared, y, s);
  return hip_status(e);
}

}  // extern "C"
