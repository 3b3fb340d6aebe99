// C ABI of the MoE decode library: host-side validation, workspace layout
// and kernel sequencing.  Semantics of every entry point are documented in
// include/moe.h.
#include "../../include/moe.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "moe_internal.h"

// Scratch of moe_decode_layer_noalloc: one array per GPU, held until the
// process ends.  Host code never uses its name as an address (on the host
// it only stands for the symbol); it uses the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

using moe::LayerT1;
using moe::LayerTB;

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Bump allocator over the workspace (offsets only).
struct Carver {
  size_t o = 0;
  size_t take(size_t bytes) {
    const size_t at = o;
    o += align_up(bytes);
    return at;
  }
};

// A shared expert whose FFN width differs from the routed experts'.
bool shared_apart(const moe_shape& s) { return s.n_shared && s.shared_ffn != s.ffn; }

// Single-token layout.
struct WsT1 {
  size_t reserved, logits, idx, wts, act_hl, act_sh, part_sh, part, xn, total;
};

WsT1 ws_t1(const moe_shape& s) {
  WsT1 L{};
  Carver c;
  const size_t nslot = (size_t)s.top_k + (size_t)s.n_shared;
  const bool apart = shared_apart(s);
  L.reserved = c.take(MOE_WS_COUNTER_BYTES);
  L.logits = c.take(sizeof(float) * s.n_experts);
  L.idx = c.take(sizeof(int32_t) * s.top_k);
  L.wts = c.take(sizeof(float) * s.top_k);
  L.act_hl = c.take(sizeof(uint16_t) * 2 * (apart ? (size_t)s.top_k : nslot) * s.ffn);
  L.act_sh = apart ? c.take(sizeof(uint16_t) * 2 * (size_t)s.shared_ffn) : 0;
  L.part_sh = apart ? c.take(sizeof(float) * s.hidden) : 0;
  L.part = c.take(sizeof(float) * nslot * s.hidden);
  L.xn = c.take(sizeof(uint16_t) * s.hidden);
  L.total = c.o;
  return L;
}

// Grouping part of the batched layout (also used by moe_group_by_expert).
struct WsGroup {
  size_t ginfo, g_expert, g_start, g_count, order, pos_of;
};

WsGroup ws_group(Carver& c, int E, int T, int k) {
  WsGroup G{};
  const size_t P = (size_t)T * k;
  G.ginfo = c.take(4 * sizeof(int32_t));
  G.g_expert = c.take(sizeof(int32_t) * (E + 1));
  G.g_start = c.take(sizeof(int32_t) * (E + 1));
  G.g_count = c.take(sizeof(int32_t) * (E + 1));
  G.order = c.take(sizeof(int32_t) * (P + T));
  G.pos_of = c.take(sizeof(int32_t) * P);
  return G;
}

// Batched (T >= 2) layout.
struct WsTB {
  size_t reserved, part, idx, wts, act_hi, act_lo, act_sh_hi, act_sh_lo, y, xn, pass_group, pass_n0, total;
  WsGroup grp;
};

// Passes of at most 16 pairs over all groups: at most one per group plus
// one per 16 pairs.
size_t max_passes(const moe_shape& s, int T) {
  return (size_t)s.n_experts + 1 + ((size_t)T * (s.top_k + s.n_shared) + 15) / 16;
}

WsTB ws_tb(const moe_shape& s, int T) {
  WsTB L{};
  Carver c;
  const size_t P = (size_t)T * s.top_k;
  const size_t npos = P + (size_t)s.n_shared * T;
  L.reserved = c.take(MOE_WS_COUNTER_BYTES);
  L.part = c.take(sizeof(float) * moe::router_splits(s.hidden) * T * s.n_experts);
  L.idx = c.take(sizeof(int32_t) * P);
  L.wts = c.take(sizeof(float) * P);
  L.grp = ws_group(c, s.n_experts, T, s.top_k);
  // a shared expert of its own width keeps its activations apart: [T][Fs]
  const bool apart = shared_apart(s);
  const size_t nrow = apart ? P : npos;
  L.act_hi = c.take(sizeof(uint16_t) * nrow * s.ffn);
  L.act_lo = c.take(sizeof(uint16_t) * nrow * s.ffn);
  L.act_sh_hi = apart ? c.take(sizeof(uint16_t) * (size_t)T * s.shared_ffn) : 0;
  L.act_sh_lo = apart ? c.take(sizeof(uint16_t) * (size_t)T * s.shared_ffn) : 0;
  L.y = c.take(sizeof(float) * npos * s.hidden);
  L.xn = c.take(sizeof(uint16_t) * (size_t)T * s.hidden);
  L.pass_group = c.take(sizeof(int32_t) * max_passes(s, T));
  L.pass_n0 = c.take(sizeof(int32_t) * max_passes(s, T));
  L.total = c.o;
  return L;
}

size_t ws_needed(const moe_shape& s, int T) { return T <= 1 ? ws_t1(s).total : ws_tb(s, T).total; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Structural validation of a shape (no pointers).
int check_shape(const moe_shape* s) {
  if (!s) return MOE_ERR_INVALID_ARG;
  if (s->hidden <= 0 || s->n_experts <= 0 || s->top_k <= 0 || s->ffn <= 0 || s->n_shared < 0)
    return MOE_ERR_INVALID_ARG;
  if (s->top_k > s->n_experts) return MOE_ERR_INVALID_ARG;
  if (s->n_shared > 1) return MOE_ERR_UNSUPPORTED;
  if (s->n_shared == 1 && (s->shared_ffn <= 0 || s->shared_ffn % 128 || s->shared_ffn > moe::kMaxFfn))
    return s->shared_ffn <= 0 ? MOE_ERR_INVALID_ARG : MOE_ERR_UNSUPPORTED;
  if (s->n_experts > moe::kMaxExperts || s->top_k > moe::kMaxTopK) return MOE_ERR_UNSUPPORTED;
  if (s->hidden % 256 || s->hidden > 8192) return MOE_ERR_UNSUPPORTED;
  if (moe::gateup_map(s->hidden).bpl > moe::kMaxBplGateUp) return MOE_ERR_UNSUPPORTED;
  if (s->ffn % 128 || s->ffn > moe::kMaxFfn) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int check_tokens(int32_t T) {
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (T > moe::kMaxTokens) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int check_ws(const moe_shape* s, int32_t T, const void* ws, size_t ws_bytes) {
  if (!ws || !aligned16(ws)) return MOE_ERR_WORKSPACE;
  if (ws_needed(*s, T) > ws_bytes) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

int check_mat(const moe_mx_mat& m) {
  if (!m.codes || !m.scales || !aligned16(m.codes)) return MOE_ERR_INVALID_ARG;
  if ((uintptr_t)m.scales & 3u) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

int check_weights(const moe_shape* s, const moe_layer_weights* w, bool need_router) {
  if (!w) return MOE_ERR_INVALID_ARG;
  if (need_router && (!w->router_w || !aligned16(w->router_w))) return MOE_ERR_INVALID_ARG;
  int rc;
  if ((rc = check_mat(w->gate)) || (rc = check_mat(w->up)) || (rc = check_mat(w->down))) return rc;
  if (s->n_shared &&
      ((rc = check_mat(w->s_gate)) || (rc = check_mat(w->s_up)) || (rc = check_mat(w->s_down))))
    return rc;
  return MOE_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

template <class Layer>
void set_weights(Layer& L, const moe_shape* s, const moe_layer_weights* w) {
  if (!w) return;
  L.router_w = w->router_w;
  L.g_codes = w->gate.codes;
  L.g_scales = w->gate.scales;
  L.u_codes = w->up.codes;
  L.u_scales = w->up.scales;
  L.d_codes = w->down.codes;
  L.d_scales = w->down.scales;
  if (s->n_shared) {
    L.sg_codes = w->s_gate.codes;
    L.sg_scales = w->s_gate.scales;
    L.su_codes = w->s_up.codes;
    L.su_scales = w->s_up.scales;
    L.sd_codes = w->s_down.codes;
    L.sd_scales = w->s_down.scales;
  }
}

LayerT1 make_layer(const moe_shape* s, const moe_layer_weights* w, void* ws) {
  const WsT1 W = ws_t1(*s);
  char* b = (char*)ws;
  LayerT1 L{};
  L.H = s->hidden;
  L.E = s->n_experts;
  L.k = s->top_k;
  L.F = s->ffn;
  L.S = s->n_shared;
  L.Fs = s->n_shared ? s->shared_ffn : s->ffn;
  set_weights(L, s, w);
  L.logits = (float*)(b + W.logits);
  L.act_sh = shared_apart(*s) ? (uint16_t*)(b + W.act_sh) : nullptr;
  L.part_sh = shared_apart(*s) ? (float*)(b + W.part_sh) : nullptr;
  L.idx = (int32_t*)(b + W.idx);
  L.wts = (float*)(b + W.wts);
  L.act_hl = (uint16_t*)(b + W.act_hl);
  L.part = (float*)(b + W.part);
  L.counters = (uint32_t*)(b + W.reserved);
  L.xn = (uint16_t*)(b + W.xn);
  return L;
}

void set_group(LayerTB& L, const WsGroup& G, char* b) {
  L.ginfo = (int32_t*)(b + G.ginfo);
  L.g_expert = (int32_t*)(b + G.g_expert);
  L.g_start = (int32_t*)(b + G.g_start);
  L.g_count = (int32_t*)(b + G.g_count);
  L.order = (int32_t*)(b + G.order);
  L.pos_of = (int32_t*)(b + G.pos_of);
}

LayerTB make_layer_tb(const moe_shape* s, const moe_layer_weights* w, void* ws, int T) {
  const WsTB W = ws_tb(*s, T);
  char* b = (char*)ws;
  LayerTB L{};
  L.T = T;
  L.H = s->hidden;
  L.E = s->n_experts;
  L.k = s->top_k;
  L.F = s->ffn;
  L.S = s->n_shared;
  L.KS = moe::router_splits(s->hidden);
  set_weights(L, s, w);
  L.part = (float*)(b + W.part);
  L.idx = (int32_t*)(b + W.idx);
  L.wts = (float*)(b + W.wts);
  set_group(L, W.grp, b);
  L.pass_group = (int32_t*)(b + W.pass_group);
  L.pass_n0 = (int32_t*)(b + W.pass_n0);
  L.act_hi = (uint16_t*)(b + W.act_hi);
  L.act_lo = (uint16_t*)(b + W.act_lo);
  L.Fs = s->n_shared ? s->shared_ffn : s->ffn;
  if (shared_apart(*s)) {
    L.act_sh_hi = (uint16_t*)(b + W.act_sh_hi);
    L.act_sh_lo = (uint16_t*)(b + W.act_sh_lo);
  }
  L.y = (float*)(b + W.y);
  return L;
}

uint16_t* xn_tb(const moe_shape* s, void* ws, int T) { return (uint16_t*)((char*)ws + ws_tb(*s, T).xn); }

// One full single-token layer: K1a (router), K2 (top-k, shared + routed
// gate/up), K3 (down of every slot + combine) on one stream.
int run_layer_t1(LayerT1& L, hipStream_t st) { return hip_status(moe::launch_layer_t1(L, st)); }

// One batched layer: router, top-k, grouping, gate/up, down, combine.  A
// shared expert of its own width (its group holds every token, last in the
// grouping) runs its gate/up and down as passes of their own, at width Fs,
// with its activations in their own planes; its outputs land in the same
// per-pair rows, so the combine is unchanged.
int run_layer_tb(LayerTB& L, hipStream_t st) {
  if (moe::launch_router_tb(L, st) != hipSuccess) return MOE_ERR_HIP;
  if (moe::launch_topk_tb(L, st) != hipSuccess) return MOE_ERR_HIP;
  if (moe::launch_group_tb(L, st) != hipSuccess) return MOE_ERR_HIP;
  if (L.S && L.act_sh_hi) {
    LayerTB Lr = L;  // routed groups
    Lr.gmode = 1;
    LayerTB Ls = L;  // the shared group, at its own width
    Ls.gmode = 2;
    Ls.F = L.Fs;
    Ls.act_hi = L.act_sh_hi;
    Ls.act_lo = L.act_sh_lo;
    Ls.pos0 = L.T * L.k;
    if (moe::launch_gateup_tb(Lr, st) != hipSuccess) return MOE_ERR_HIP;
    if (moe::launch_gateup_tb(Ls, st) != hipSuccess) return MOE_ERR_HIP;
    if (moe::launch_down_tb(Lr, st) != hipSuccess) return MOE_ERR_HIP;
    if (moe::launch_down_tb(Ls, st) != hipSuccess) return MOE_ERR_HIP;
    return hip_status(moe::launch_combine_tb(L, st));
  }
  if (moe::launch_gateup_tb(L, st) != hipSuccess) return MOE_ERR_HIP;
  if (moe::launch_down_tb(L, st) != hipSuccess) return MOE_ERR_HIP;
  return hip_status(moe::launch_combine_tb(L, st));
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or size";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int moe_workspace_size(const moe_shape* shape, int32_t max_tokens, size_t* bytes) {
  int rc;
  if ((rc = check_shape(shape)) || (rc = check_tokens(max_tokens))) return rc;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  size_t n = ws_t1(*shape).total;
  if (max_tokens >= 2) {
    const size_t m = ws_tb(*shape, max_tokens).total;
    n = m > n ? m : n;
  }
  *bytes = n;
  return MOE_OK;
}

int moe_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws || !aligned16(ws)) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_zero_fill(ws, ws_bytes & ~(size_t)3, (hipStream_t)stream));
}

int moe_router_topk(const moe_shape* shape, const uint16_t* x, const uint16_t* router_w,
                    int32_t n_tokens, int32_t* topk_idx, float* topk_w, float* logits, void* ws,
                    size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_shape(shape)) || (rc = check_tokens(n_tokens))) return rc;
  if (n_tokens == 0) return MOE_OK;
  if (!x || !aligned16(x) || !router_w || !aligned16(router_w) || !topk_idx || !topk_w)
    return MOE_ERR_INVALID_ARG;
  if ((rc = check_ws(shape, n_tokens, ws, ws_bytes))) return rc;
  const hipStream_t st = (hipStream_t)stream;
  if (n_tokens == 1) {
    LayerT1 L = make_layer(shape, nullptr, ws);
    L.router_w = router_w;
    L.x = x;
    L.idx_out = topk_idx;
    L.w_out = topk_w;
    L.logits_out = logits;
    if (moe::launch_router_t1(L, st) != hipSuccess) return MOE_ERR_HIP;
    return hip_status(moe::launch_topk_t1(L, st));
  }
  LayerTB L = make_layer_tb(shape, nullptr, ws, n_tokens);
  L.router_w = router_w;
  L.x = x;
  L.idx_out = topk_idx;
  L.w_out = topk_w;
  L.logits_out = logits;
  if (moe::launch_router_tb(L, st) != hipSuccess) return MOE_ERR_HIP;
  return hip_status(moe::launch_topk_tb(L, st));
}

int moe_expert_gateup(const moe_shape* shape, const moe_layer_weights* w, const uint16_t* x,
                      const int32_t* topk_idx, int32_t n_tokens, float* act, void* ws,
                      size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_shape(shape)) || (rc = check_tokens(n_tokens))) return rc;
  if (n_tokens == 0) return MOE_OK;
  if ((rc = check_weights(shape, w, false))) return rc;
  if (!x || !aligned16(x) || !topk_idx || !act) return MOE_ERR_INVALID_ARG;
  if ((rc = check_ws(shape, n_tokens, ws, ws_bytes))) return rc;
  if (n_tokens > 1) return MOE_ERR_UNSUPPORTED;
  LayerT1 L = make_layer(shape, w, ws);
  return hip_status(moe::launch_gateup_t1(L, x, topk_idx, act, false, (hipStream_t)stream));
}

}  // extern "C"

namespace {

int decode_layer(const moe_shape* shape, const moe_layer_weights* w, const uint16_t* x,
                 const uint16_t* residual, uint16_t* out, int32_t n_tokens,
                 int32_t* topk_idx_out, float* topk_w_out, void* ws, size_t ws_bytes,
                 void* stream, moe::KernelTimer* timer) {
  int rc;
  if ((rc = check_shape(shape)) || (rc = check_tokens(n_tokens))) return rc;
  if (n_tokens == 0) return MOE_OK;
  if ((rc = check_weights(shape, w, true))) return rc;
  if (!x || !aligned16(x) || !out || !aligned16(out)) return MOE_ERR_INVALID_ARG;
  if (residual && !aligned16(residual)) return MOE_ERR_INVALID_ARG;
  const size_t vec = sizeof(uint16_t) * (size_t)n_tokens * shape->hidden;
  if (residual != x && overlaps(out, vec, x, vec)) return MOE_ERR_INVALID_ARG;
  if (residual && residual != out && overlaps(out, vec, residual, vec)) return MOE_ERR_INVALID_ARG;
  if ((rc = check_ws(shape, n_tokens, ws, ws_bytes))) return rc;
  if (overlaps(ws, ws_bytes, out, vec) || overlaps(ws, ws_bytes, x, vec)) return MOE_ERR_INVALID_ARG;
  const hipStream_t st = (hipStream_t)stream;
  if (n_tokens == 1) {
    LayerT1 L = make_layer(shape, w, ws);
    L.x = x;
    L.residual = residual;
    L.out = out;
    L.idx_out = topk_idx_out;
    L.w_out = topk_w_out;
    L.timer = timer;
    return run_layer_t1(L, st);
  }
  LayerTB L = make_layer_tb(shape, w, ws, n_tokens);
  L.x = x;
  L.residual = residual;
  L.out = out;
  L.idx_out = topk_idx_out;
  L.w_out = topk_w_out;
  L.timer = timer;
  return run_layer_tb(L, st);
}

}  // namespace

extern "C" {

int moe_decode_layer(const moe_shape* shape, const moe_layer_weights* w, const uint16_t* x,
                     const uint16_t* residual, uint16_t* out, int32_t n_tokens,
                     int32_t* topk_idx_out, float* topk_w_out, void* ws, size_t ws_bytes,
                     void* stream) {
  return decode_layer(shape, w, x, residual, out, n_tokens, topk_idx_out, topk_w_out, ws,
                      ws_bytes, stream, nullptr);
}

int moe_decode_layer_timed(const moe_shape* shape, const moe_layer_weights* w, const uint16_t* x,
                           const uint16_t* residual, uint16_t* out, int32_t n_tokens,
                           int32_t* topk_idx_out, float* topk_w_out, void* ws, size_t ws_bytes,
                           void* stream, void* const* events, int32_t max_kernels,
                           int32_t* n_kernels) {
  if (!events || max_kernels < 0 || max_kernels > MOE_MAX_LAYER_KERNELS || !n_kernels)
    return MOE_ERR_INVALID_ARG;
  hipEvent_t start[MOE_MAX_LAYER_KERNELS], stop[MOE_MAX_LAYER_KERNELS];
  for (int i = 0; i < max_kernels; ++i) {
    start[i] = (hipEvent_t)events[2 * i];
    stop[i] = (hipEvent_t)events[2 * i + 1];
    if (!start[i] || !stop[i]) return MOE_ERR_INVALID_ARG;
  }
  moe::KernelTimer tm{start, stop, max_kernels, 0};
  *n_kernels = 0;
  const int rc = decode_layer(shape, w, x, residual, out, n_tokens, topk_idx_out, topk_w_out, ws,
                              ws_bytes, stream, &tm);
  if (rc == MOE_OK) *n_kernels = tm.used;
  return rc;
}

}  // extern "C"

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device, once resolved

// The current device's scratch address; on the first call for a device it is
// looked up and the counter head is cleared by a fill kernel on `st`.
int scratch_of_current_device(hipStream_t st, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    if (moe::launch_zero_fill(p, MOE_WS_COUNTER_BYTES, st) != hipSuccess) return MOE_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_decode_layer_noalloc(const moe_shape* shape, const moe_layer_weights* w, const uint16_t* x,
                             const uint16_t* residual, uint16_t* out, int32_t n_tokens,
                             int32_t* topk_idx_out, float* topk_w_out, void* stream) {
  int rc;
  if ((rc = check_shape(shape)) || (rc = check_tokens(n_tokens))) return rc;
  if (n_tokens == 0) return MOE_OK;
  if (ws_needed(*shape, n_tokens) > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if ((rc = scratch_of_current_device((hipStream_t)stream, &ws))) return rc;
  return decode_layer(shape, w, x, residual, out, n_tokens, topk_idx_out, topk_w_out, ws,
                      (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

int moe_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || !aligned16(buf) || (bytes & 15u)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_stream_read(buf, bytes, sink, (hipStream_t)stream));
}

int moe_decode_stack(const moe_shape* shape, const moe_layer_weights* layers,
                     const uint16_t* const* gammas, float eps, int32_t n_layers, uint16_t* hidden,
                     int32_t n_tokens, int32_t* topk_idx_out, uint16_t* hidden_trace, void* ws,
                     size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_shape(shape)) || (rc = check_tokens(n_tokens))) return rc;
  if (n_layers < 0 || !(eps >= 0.0f)) return MOE_ERR_INVALID_ARG;
  if (n_tokens == 0 || n_layers == 0) return MOE_OK;
  if (!layers || !gammas || !hidden || !aligned16(hidden)) return MOE_ERR_INVALID_ARG;
  for (int l = 0; l < n_layers; ++l) {
    if ((rc = check_weights(shape, &layers[l], true))) return rc;
    if (!gammas[l] || !aligned16(gammas[l])) return MOE_ERR_INVALID_ARG;
  }
  if (hidden_trace && !aligned16(hidden_trace)) return MOE_ERR_INVALID_ARG;
  if ((rc = check_ws(shape, n_tokens, ws, ws_bytes))) return rc;
  const size_t vec = sizeof(uint16_t) * (size_t)n_tokens * shape->hidden;
  if (overlaps(ws, ws_bytes, hidden, vec)) return MOE_ERR_INVALID_ARG;
  const hipStream_t st = (hipStream_t)stream;
  for (int l = 0; l < n_layers; ++l) {
    uint16_t* trace = hidden_trace ? hidden_trace + (size_t)l * n_tokens * shape->hidden : nullptr;
    int32_t* idx_out = topk_idx_out ? topk_idx_out + (size_t)l * n_tokens * shape->top_k : nullptr;
    if (n_tokens == 1) {
      LayerT1 L = make_layer(shape, &layers[l], ws);
      L.x = hidden;
      L.gamma = gammas[l];
      L.eps = eps;
      L.residual = hidden;
      L.out = hidden;
      L.trace = trace;
      L.idx_out = idx_out;
      if ((rc = run_layer_t1(L, st))) return rc;
    } else {
      uint16_t* xn = xn_tb(shape, ws, n_tokens);
      if (moe::launch_rmsnorm_tb(hidden, gammas[l], eps, n_tokens, shape->hidden, xn, st) !=
          hipSuccess)
        return MOE_ERR_HIP;
      LayerTB L = make_layer_tb(shape, &layers[l], ws, n_tokens);
      L.x = xn;
      L.residual = hidden;
      L.out = hidden;
      L.trace = trace;
      L.idx_out = idx_out;
      if ((rc = run_layer_tb(L, st))) return rc;
    }
  }
  return MOE_OK;
}

int moe_group_by_expert(const int32_t* topk_idx, int32_t n_tokens, int32_t top_k,
                        int32_t n_experts, int32_t* offsets, int32_t* pairs, void* ws,
                        size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_tokens(n_tokens))) return rc;
  if (top_k <= 0 || n_experts <= 0 || top_k > n_experts) return MOE_ERR_INVALID_ARG;
  if (top_k > moe::kMaxTopK || n_experts > moe::kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (n_tokens == 0) return MOE_OK;
  if (!topk_idx || !offsets || !pairs) return MOE_ERR_INVALID_ARG;
  if (!ws || !aligned16(ws)) return MOE_ERR_WORKSPACE;
  // the tables start after the counter head, as in the layer's own layout,
  // so that the counters other calls rely on stay at zero
  Carver c;
  c.take(MOE_WS_COUNTER_BYTES);
  const WsGroup G = ws_group(c, n_experts, n_tokens, top_k);
  if (c.o > ws_bytes) return MOE_ERR_WORKSPACE;
  LayerTB L{};
  L.T = n_tokens;
  L.E = n_experts;
  L.k = top_k;
  L.S = 0;
  L.idx = const_cast<int32_t*>(topk_idx);
  set_group(L, G, (char*)ws);
  L.offsets_out = offsets;
  L.pairs_out = pairs;
  return hip_status(moe::launch_group_tb(L, (hipStream_t)stream));
}

}  // extern "C"
