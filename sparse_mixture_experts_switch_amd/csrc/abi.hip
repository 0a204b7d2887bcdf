// C ABI of the Switch layer forward: host-side validation, workspace carving
// and the stream-ordered launch sequence.  The contract of every entry point
// is documented in include/switch_moe.h.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <exception>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/switch_moe.h"
#include "launch.h"

using namespace smx;

// Workspace of switch_layer_forward_noalloc: a file-scope device array, one
// copy on every GPU the library runs on, held until the process ends.  Host
// code never uses its name as a device address: each device's address comes
// from hipGetSymbolAddress (scratch_address).
constexpr size_t kNoAllocScratchBytes = size_t(1) << 27;  // 128 MiB
__device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char *what) {
  return fail(SWITCH_E_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

// Debug mode: with the environment variable SMX_DEBUG_SYNC set to anything
// but "" or "0" (read once, at the first launch), every entry point waits for
// its stream after each kernel it launches and fails with that kernel's name
// when the wait reports an error, so a fault is pinned to the kernel that
// raised it instead of surfacing at some later call.
bool debug_sync() {
  static const bool on = [] {
    const char *v = std::getenv("SMX_DEBUG_SYNC");
    return v && *v && std::strcmp(v, "0") != 0;
  }();
  return on;
}

// Result of a single-kernel entry point: the launch status, then, in debug
// mode, the status of a wait for the stream.
int launched(hipError_t e, const char *what, void *stream) {
  if (e != hipSuccess) return hip_fail(e, what);
  if (debug_sync() && (e = hipStreamSynchronize((hipStream_t)stream)) != hipSuccess)
    return fail(SWITCH_E_HIP, "%s (SMX_DEBUG_SYNC wait): %s (%d)", what, hipGetErrorString(e), (int)e);
  return SWITCH_OK;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; null with the error text set
// when the lookup fails.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

void *scratch_address() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    hip_fail(e, "hipGetDevice");
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    fail(SWITCH_E_HIP, "device %d beyond the %d the no-allocation workspace serves", dev, kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

constexpr size_t kWsAlign = 256;

size_t align_up(size_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }

// Products of non-negative sizes; false on overflow past 2^62.
bool mul(size_t &out, std::initializer_list<int64_t> xs) {
  unsigned __int128 p = 1;
  for (int64_t x : xs) {
    if (x < 0) return false;
    p *= (unsigned __int128)x;
    if (p > ((unsigned __int128)1 << 62)) return false;
  }
  out = (size_t)p;
  return true;
}

int esize(int dtype) { return dtype == SWITCH_BF16 ? 2 : 4; }

struct Layout {
  size_t bcount = 0, boff = 0, ppart = 0, psum = 0, rank = 0, logits = 0, wplanes = 0, route_end = 0;
  size_t fz_sync = 0, fz_aggc = 0, fz_aggp = 0, fz_incc = 0, fz_incp = 0;  // single-pass routing
  size_t fz_clear = 0;
  int64_t fz_stride = 0;
  size_t ffn_hidden = 0, ffn_end = 0;                           // switch_expert_ffn alone
  size_t lf_hidden = 0, lf_tok = 0, lf_gmap = 0, total = 0;     // layer forward
  size_t lf_rows = 0, lf_routed = 0;                            // top-k layer forward (k > 1)
};

int check_shape(const switch_shape *s) {
  if (!s) return fail(SWITCH_E_INVALID, "shape is NULL");
  if (s->tokens < 0) return fail(SWITCH_E_INVALID, "tokens = %lld < 0", (long long)s->tokens);
  if (s->d_model < 1 || s->d_ff < 1 || s->num_experts < 1)
    return fail(SWITCH_E_INVALID, "d_model = %d, d_ff = %d, num_experts = %d must be >= 1", s->d_model, s->d_ff,
                s->num_experts);
  if (s->capacity < 0) return fail(SWITCH_E_INVALID, "capacity = %d < 0", s->capacity);
  if (s->dtype != SWITCH_F32 && s->dtype != SWITCH_BF16) return fail(SWITCH_E_INVALID, "dtype = %d", s->dtype);
  if (s->tokens > INT32_MAX)
    return fail(SWITCH_E_UNSUPPORTED, "tokens = %lld above 2^31-1", (long long)s->tokens);
  if (s->d_model % 64 || s->d_ff % 64)
    return fail(SWITCH_E_UNSUPPORTED, "d_model = %d and d_ff = %d must be multiples of 64", s->d_model, s->d_ff);
  if (s->weight_layout != SWITCH_WEIGHTS_ROWS && s->weight_layout != SWITCH_WEIGHTS_TILED)
    return fail(SWITCH_E_INVALID, "weight_layout = %d", s->weight_layout);
  if (s->weight_layout == SWITCH_WEIGHTS_TILED && s->dtype != SWITCH_BF16)
    return fail(SWITCH_E_UNSUPPORTED, "tiled expert weights are bf16 only");
  return SWITCH_OK;
}

bool tiled(const switch_shape *s) { return s->weight_layout == SWITCH_WEIGHTS_TILED; }

// Workspace of a call with k routes per token: the router's per-block
// partials (k blocks per router block), the route ranks, the logits rows when
// the experts do not fit one chunk, W_r's bf16 planes (bf16 layers with
// row-major weights), then the
// layer's hidden activations and
// slot maps; k > 1 adds the slot -> output row map and the [k][T][d] buffer of
// gate-scaled expert outputs per route.
int layout(const switch_shape *s, Layout &L, int k = 1) {
  const int64_t T = s->tokens, N = s->num_experts, C = s->capacity, d = s->d_model, f = s->d_ff;
  const int64_t nb = router_blocks(T) * k, Tp = router_blocks(T) * kRouterTokens * k;
  const int es = esize(s->dtype);
  size_t bc, pp, ps, rk, lg = 0, hid, act, tk, rt = 0, sy, r32, r64;
  // tiled weights: the caller's W_r argument already holds the planes
  const size_t wpl =
      s->dtype == SWITCH_BF16 && s->weight_layout != SWITCH_WEIGHTS_TILED ? (size_t)router_planes_bytes((int)N, (int)d)
                                                                          : 0;
  const int64_t Np = count_stride((int)N), Ns = (N + 63) / 64 * 64;
  bool ok = mul(bc, {nb, Np, 4}) && mul(pp, {nb, Np, 4}) && mul(ps, {N, 4}) && mul(rk, {Tp, 4}) &&
            mul(sy, {nb + 4, 4}) && mul(r32, {nb, Ns, 4}) && mul(r64, {nb, Ns, 8}) &&
            (N <= kRouterChunk || mul(lg, {T, N, 4})) && mul(hid, {N, C, f, es}) && mul(act, {N, C, d, es}) &&
            mul(tk, {N, C, 4}) && (k == 1 || mul(rt, {k, T, d, es}));
  if (!ok) return fail(SWITCH_E_UNSUPPORTED, "buffer sizes overflow for this shape");
  size_t o = 0;
  L.bcount = o;
  o = align_up(o + bc);
  L.boff = o;
  o = align_up(o + bc);
  L.ppart = o;
  o = align_up(o + pp);
  L.psum = o;
  o = align_up(o + ps);
  L.rank = o;
  o = align_up(o + rk);
  L.logits = o;
  o = align_up(o + lg);
  L.wplanes = o;
  o = align_up(o + wpl);
  L.fz_sync = o;  // ticket, error word and block states; then the look-back rows
  L.fz_clear = (sy + 15) / 16 * 16;
  o = align_up(o + sy);
  L.fz_stride = Ns;
  L.fz_aggc = o;
  o = align_up(o + r32);
  L.fz_incc = o;
  o = align_up(o + r32);
  L.fz_aggp = o;
  o = align_up(o + r64);
  L.fz_incp = o;
  o = align_up(o + r64);
  L.route_end = o;
  L.ffn_hidden = 0;
  L.ffn_end = align_up(hid);
  L.lf_hidden = o;
  o = align_up(o + hid);
  L.lf_tok = o;
  o = align_up(o + tk);
  L.lf_gmap = o;
  o = align_up(o + tk);
  if (k > 1) {
    L.lf_rows = o;
    o = align_up(o + tk);
    L.lf_routed = o;
    o = align_up(o + rt);
  }
  L.total = o;
  return SWITCH_OK;
}

// Routes per token: 1 (Switch routing) or 2 (classic top-2), at most N, and
// k * tokens rows must be indexable by int32.
int check_topk(const switch_shape *s, int32_t top_k) {
  if (top_k < 1) return fail(SWITCH_E_INVALID, "top_k = %d < 1", top_k);
  if (top_k > s->num_experts)
    return fail(SWITCH_E_INVALID, "top_k = %d above num_experts = %d", top_k, s->num_experts);
  if (top_k > 2) return fail(SWITCH_E_UNSUPPORTED, "top_k = %d: only 1 and 2 are supported", top_k);
  if ((int64_t)top_k * s->tokens > INT32_MAX)
    return fail(SWITCH_E_UNSUPPORTED, "top_k x tokens = %lld above 2^31-1", (long long)top_k * s->tokens);
  return SWITCH_OK;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

#define NEED(ptr, al)                                                                            \
  do {                                                                                           \
    if (!(ptr)) return fail(SWITCH_E_INVALID, "%s is NULL", #ptr);                               \
    if (!aligned((ptr), (al))) return fail(SWITCH_E_INVALID, "%s is not %d-byte aligned", #ptr, (int)(al)); \
  } while (0)

#define GUARD(...)                                            \
  try {                                                       \
    __VA_ARGS__                                               \
  } catch (const std::exception &ex) {                        \
    return fail(SWITCH_E_HIP, "internal error: %s", ex.what()); \
  } catch (...) {                                             \
    return fail(SWITCH_E_HIP, "internal error");              \
  }

int check_ws(void *ws, size_t ws_bytes, size_t need) {
  if (need == 0) return SWITCH_OK;
  if (!ws) return fail(SWITCH_E_INVALID, "workspace is NULL");
  if (!aligned(ws, kWsAlign)) return fail(SWITCH_E_INVALID, "workspace is not 256-byte aligned");
  if (ws_bytes < need)
    return fail(SWITCH_E_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);
  return SWITCH_OK;
}

// ---------------------------------------------------------------- launches --
// Launch sequence control: records the name of each kernel in launch order
// and says how many times to issue it: once, or, for a measurement call, only
// the kernels numbered first..last, each `times` times back to back (every
// kernel of the layer reads only what earlier kernels wrote and never its own
// outputs, so a repeat or a rerun on the same workspace changes no result).
// In debug mode each mark also waits for the stream; after a failed wait no
// further kernel is issued and done() turns the call's result into the error.
struct Timer {
  int first = 0, last = 1 << 30;
  int times = 1;
  int n = 0;  // kernels of this call passed so far
  const char *names[16] = {};
  hipStream_t st = nullptr;
  hipError_t err = hipSuccess;  // debug mode: first failed wait
  const char *bad = nullptr;    // debug mode: the kernel before it
  explicit Timer(void *stream) : st((hipStream_t)stream) {}
  int reps() const { return (err == hipSuccess && n >= first && n <= last) ? times : 0; }
  void mark(const char *name) {
    if (n < 16) names[n] = name;
    ++n;
    if (err == hipSuccess && debug_sync()) {
      hipError_t e = hipStreamSynchronize(st);
      if (e != hipSuccess) {
        err = e;
        bad = name;
      }
    }
  }
  int done(int rc) const {
    if (rc == SWITCH_OK && err != hipSuccess)
      return fail(SWITCH_E_HIP, "kernel %s (SMX_DEBUG_SYNC wait): %s (%d)", bad, hipGetErrorString(err), (int)err);
    return rc;
  }
};

constexpr int kNumKernels = 5;  // most launches one call makes

int route_args(const switch_shape *s, const void *x, const float *w_router, const float *router_bias,
               int32_t *expert_idx, float *gate, int32_t *slot, uint8_t *dropped, int32_t *expert_count,
               float *aux_loss, void *ws, size_t ws_bytes, const Layout &L, RouteArgs &a) {
  const bool any = s->tokens > 0;
  if (any) {
    NEED(x, 16);
    NEED(expert_idx, 4);
    NEED(gate, 4);
    NEED(slot, 4);
    if (!dropped) return fail(SWITCH_E_INVALID, "dropped is NULL");
  }
  NEED(w_router, 16);
  if (router_bias && !aligned(router_bias, 4)) return fail(SWITCH_E_INVALID, "router_bias is not 4-byte aligned");
  NEED(expert_count, 4);
  NEED(aux_loss, 4);
  int rc = check_ws(ws, ws_bytes, L.route_end);
  if (rc) return rc;
  char *w = (char *)ws;
  a.dtype = s->dtype;
  a.k = 1;
  a.T = s->tokens;
  a.d = s->d_model;
  a.N = s->num_experts;
  a.C = s->capacity;
  a.x = x;
  a.w_r = w_router;
  a.bias = router_bias;
  a.logits = (float *)(w + L.logits);
  a.wr_planes = tiled(s);  // W_r given as its planes (switch_tile_router)
  a.wplanes = a.wr_planes ? (void *)w_router : (void *)(w + L.wplanes);
  a.expert_idx = expert_idx;
  a.gate = gate;
  a.slot = slot;
  a.dropped = dropped;
  a.expert_count = expert_count;
  a.aux_loss = aux_loss;
  a.bcount = (int32_t *)(w + L.bcount);
  a.boff = (int32_t *)(w + L.boff);
  a.rank = (int32_t *)(w + L.rank);
  a.ppart = (float *)(w + L.ppart);
  a.psum = (float *)(w + L.psum);
  return SWITCH_OK;
}

// Routing kernels: router, then the capacity assignment (one or two
// launches).  With maps.tok set (layer path) the assignment also fills the
// slot -> token / output row / gate maps and, for one route per token, the
// output rows of dropped tokens.
int run_route(const RouteArgs &a, hipStream_t st, Timer &tm, const LayerMaps &maps = LayerMaps{}) {
  hipError_t e;
  for (int r = tm.reps(); r > 0; --r)
    if ((e = launch_router(a, st)) != hipSuccess) return hip_fail(e, "router launch");
  tm.mark("router");
  LaunchMarks marks{[](void *ctx, const char *name) { static_cast<Timer *>(ctx)->mark(name); },
                    [](void *ctx) { return static_cast<Timer *>(ctx)->reps(); }, &tm};
  if ((e = launch_assign(a, maps, st, marks)) != hipSuccess) return hip_fail(e, "assignment launch");
  return SWITCH_OK;
}

// The layer with k routes per token.  k = 1: the expert FFN's epilogue writes
// y directly.  k = 2: it writes each kept route's gate-scaled output to row
// r * T + t of a workspace buffer, and a last kernel adds the kept routes of
// each token (and x with the residual) into y.  The expert FFN is one fused
// kernel where the shape allows it, unless save_hidden asks for the hidden
// activations H in the workspace (the backward reads them): then it is the
// up-projection (writing H) and the down-projection with the combine.
bool fused_ffn(const switch_shape *s, bool save_hidden) {
  return !save_hidden && ffn_fused_eligible(s->dtype, s->d_model, s->d_ff, s->capacity);
}

// The block's Add + Normalize after the layer (k = 1): y then holds
// (v - mean) / sqrt(var + eps) * gamma + beta with v = x + layer output.
struct NormOpt {
  const float *gamma, *beta;
  float eps;
};

int layer_forward(const switch_shape *s, int32_t k, const void *x, const float *w_router,
                  const float *router_bias, const void *w_in, const void *w_out, int32_t add_residual, void *y,
                  int32_t *expert_idx, float *gate, int32_t *slot, uint8_t *dropped, int32_t *expert_count,
                  float *aux_loss, void *ws, size_t ws_bytes, void *stream, Timer &tm, bool save_hidden = false,
                  const NormOpt *norm = nullptr) {
  int rc = check_shape(s);
  if (rc) return rc;
  if ((rc = check_topk(s, k))) return rc;
  Layout L;
  if ((rc = layout(s, L, k))) return rc;
  if ((rc = check_ws(ws, ws_bytes, L.total))) return rc;
  RouteArgs ra;
  if ((rc = route_args(s, x, w_router, router_bias, expert_idx, gate, slot, dropped, expert_count, aux_loss, ws,
                       ws_bytes, L, ra)))
    return rc;
  ra.k = k;
  NEED(w_in, 16);
  NEED(w_out, 16);
  if (s->tokens > 0) NEED(y, 16);
  hipStream_t st = (hipStream_t)stream;
  char *w = (char *)ws;
  LayerMaps maps;
  maps.tok = (int32_t *)(w + L.lf_tok);
  maps.gmap = (float *)(w + L.lf_gmap);
  const void *xres = add_residual ? x : nullptr;
  const bool fused = fused_ffn(s, save_hidden);
  // normalization inside the fused kernel (kept rows) and the assignment
  // (dropped rows); otherwise the bare layer, then the Add + Normalize kernel
  const bool norm_fused = norm && fused;
  if (k == 1) {
    maps.xres = norm ? (norm_fused ? x : nullptr) : xres;
    maps.y = y;
    if (norm_fused) {
      maps.gamma = norm->gamma;
      maps.beta = norm->beta;
      maps.eps = norm->eps;
    }
  } else {
    maps.rows = (int32_t *)(w + L.lf_rows);
  }
  if ((rc = run_route(ra, st, tm, maps))) return rc;
  hipError_t e;
  void *routed = k == 1 ? y : (void *)(w + L.lf_routed);
  if (fused) {
    // the whole expert FFN and the combine in one kernel
    FusedFfnCall fc{s->dtype, s->num_experts, s->capacity, s->d_model, s->d_ff, x, w_in, w_out, routed,
                    expert_count, maps.tok, k == 1 ? nullptr : maps.rows, maps.gmap,
                    k == 1 ? (norm_fused ? x : xres) : nullptr};
    fc.tiled = tiled(s);
    if (norm_fused) {
      fc.gamma = norm->gamma;
      fc.beta = norm->beta;
      fc.eps = norm->eps;
    }
    for (int r = tm.reps(); r > 0; --r)
      if ((e = launch_ffn_fused(fc, st)) != hipSuccess) return hip_fail(e, "ffn launch");
    tm.mark("ffn");
  } else {
  GemmCall up{s->dtype, s->num_experts, s->capacity, s->d_model, s->d_ff, x, w_in, w + L.lf_hidden,
              expert_count, maps.tok, nullptr, nullptr, nullptr, tiled(s)};
  for (int r = tm.reps(); r > 0; --r)
    if ((e = launch_ffn_up_gather(up, st)) != hipSuccess) return hip_fail(e, "ffn_up launch");
  tm.mark("ffn_up");
  GemmCall down{s->dtype, s->num_experts, s->capacity, s->d_ff, s->d_model, w + L.lf_hidden, w_out, routed,
                expert_count, k == 1 ? maps.tok : maps.rows, gate, maps.gmap, k == 1 && !norm ? xres : nullptr,
                tiled(s)};
  down.out_rows = (int64_t)k * s->tokens;
  for (int r = tm.reps(); r > 0; --r)
    if ((e = launch_ffn_down_combine(down, st)) != hipSuccess) return hip_fail(e, "ffn_down launch");
  tm.mark("ffn_down");
  }
  if (norm && !norm_fused && s->tokens > 0) {  // in place: y = Add + Normalize(x, y)
    AddNormArgs an{s->dtype, s->tokens, s->d_model, x, y, norm->gamma, norm->beta, norm->eps, y, CombineRows{}};
    for (int r = tm.reps(); r > 0; --r)
      if ((e = launch_add_norm(an, st)) != hipSuccess) return hip_fail(e, "add_norm launch");
    tm.mark("add_norm");
  }
  if (k > 1) {
    TopkSumArgs sa{s->dtype, k, s->tokens, s->d_model, routed, dropped, xres, y};
    for (int r = tm.reps(); r > 0; --r)
      if ((e = launch_topk_sum(sa, st)) != hipSuccess) return hip_fail(e, "topk_sum launch");
    tm.mark("topk_sum");
  }
  return SWITCH_OK;
}

// Workspace of switch_layer_backward: du [N][C][d_ff], the per-token partial
// dots [T][n_dg], the experts' part of dx [T][d] (fp32), dL/dh [T][N], the
// logits scratch when N > kRouterChunk, W_r's bf16 planes for the logits
// (bf16 layers), the split partial sums of dW_r and the bias gradient, and the
// bf16 planes of the dx product.
struct BwdLayout {
  size_t du = 0, dgpart = 0, dxe = 0, dh = 0, logits = 0, wplanes = 0, wpart = 0, bpart = 0, aplanes = 0,
         bplanes = 0, total = 0;
  int n_dg = 0, splits = 1, kp = 0;
};

int bwd_layout(const switch_shape *s, BwdLayout &B) {
  const int64_t T = s->tokens, N = s->num_experts, C = s->capacity, d = s->d_model, f = s->d_ff;
  const int es = esize(s->dtype);
  B.n_dg = bwd_dz_tiles(s->dtype, (int)f);
  B.splits = router_wgrad_split(T, (int)N, (int)d).splits;
  B.kp = router_dx_kp((int)N);
  size_t du, dg, dxe, dh, lg = 0, wp, bp, ap = 0, bq = 0;
  const bool planes = s->dtype == SWITCH_BF16;  // the MFMA dx product of bf16 layers
  const size_t wpl = planes ? (size_t)router_planes_bytes((int)N, (int)d) : 0;  // the logits' W_r planes
  bool ok = mul(du, {N, C, f, es}) && mul(dg, {T, B.n_dg, 4}) && mul(dxe, {T, d, 4}) && mul(dh, {T, N, 4}) &&
            (N <= kRouterChunk || mul(lg, {T, N, 4})) && mul(wp, {B.splits, N, d, 4}) &&
            mul(bp, {router_blocks(T), N, 4}) && (!planes || (mul(ap, {T, B.kp, 2}) && mul(bq, {B.kp, d, 2})));
  if (!ok) return fail(SWITCH_E_UNSUPPORTED, "backward buffer sizes overflow for this shape");
  size_t o = 0;
  B.du = o;
  o = align_up(o + du);
  B.dgpart = o;
  o = align_up(o + dg);
  B.dxe = o;
  o = align_up(o + dxe);
  B.dh = o;
  o = align_up(o + dh);
  B.logits = o;
  o = align_up(o + lg);
  B.wplanes = o;
  o = align_up(o + wpl);
  B.wpart = o;
  o = align_up(o + wp);
  B.bpart = o;
  o = align_up(o + bp);
  B.aplanes = o;
  o = align_up(o + ap);
  B.bplanes = o;
  o = align_up(o + bq);
  B.total = o;
  return SWITCH_OK;
}

int layer_backward(const switch_shape *s, const void *x, const float *w_router, const float *router_bias,
                   const void *w_in, const void *w_out, int32_t add_residual, const int32_t *expert_idx,
                   const uint8_t *dropped, const int32_t *expert_count, const void *fwd_ws, size_t fwd_ws_bytes,
                   const void *dy, float d_aux, void *dx, float *dw_router, float *d_router_bias, void *dw_in,
                   void *dw_out, void *ws, size_t ws_bytes, void *stream, Timer &tm) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (tiled(s)) return fail(SWITCH_E_UNSUPPORTED, "the backward reads row-major expert weights");
  if (!std::isfinite(d_aux)) return fail(SWITCH_E_INVALID, "d_aux = %g is not finite", d_aux);
  Layout L;
  if ((rc = layout(s, L))) return rc;
  BwdLayout B;
  if ((rc = bwd_layout(s, B))) return rc;
  if (!fwd_ws) return fail(SWITCH_E_INVALID, "fwd_workspace is NULL");
  if (!aligned(fwd_ws, kWsAlign)) return fail(SWITCH_E_INVALID, "fwd_workspace is not 256-byte aligned");
  if (fwd_ws_bytes < L.total)
    return fail(SWITCH_E_WORKSPACE, "fwd_workspace of %zu bytes, the forward needs %zu", fwd_ws_bytes, L.total);
  if ((rc = check_ws(ws, ws_bytes, B.total))) return rc;
  NEED(w_router, 16);
  if (router_bias && !aligned(router_bias, 4)) return fail(SWITCH_E_INVALID, "router_bias is not 4-byte aligned");
  NEED(w_in, 16);
  NEED(w_out, 16);
  NEED(expert_count, 4);
  NEED(dw_router, 16);
  if (d_router_bias && !aligned(d_router_bias, 4))
    return fail(SWITCH_E_INVALID, "d_router_bias is not 4-byte aligned");
  NEED(dw_in, 16);
  NEED(dw_out, 16);
  if (s->tokens > 0) {
    NEED(x, 16);
    NEED(dy, 16);
    NEED(dx, 16);
    NEED(expert_idx, 4);
    if (!dropped) return fail(SWITCH_E_INVALID, "dropped is NULL");
  }
  hipStream_t st = (hipStream_t)stream;
  const char *fw = (const char *)fwd_ws;
  char *w = (char *)ws;
  BwdLaunch bl{s->dtype, s->tokens, s->d_model, s->d_ff, s->num_experts, s->capacity, x, w_in, w_out, dy,
               expert_count, (const int32_t *)(fw + L.lf_tok), (const float *)(fw + L.lf_gmap),
               fw + L.lf_hidden, w + B.du, (float *)(w + B.dgpart), (float *)(w + B.dxe), dw_in, dw_out};
  LaunchMarks marks{[](void *ctx, const char *name) { static_cast<Timer *>(ctx)->mark(name); },
                    [](void *ctx) { return static_cast<Timer *>(ctx)->reps(); }, &tm};
  hipError_t e;
  if ((e = launch_bwd_experts(bl, st, marks)) != hipSuccess) return hip_fail(e, "backward expert launch");
  RouterBwdArgs ra{s->dtype, s->tokens, s->d_model, s->num_experts, x, w_router, router_bias,
                   (float *)(w + B.logits), w + B.wplanes, expert_idx, dropped, expert_count,
                   (const float *)(w + B.dgpart),
                   B.n_dg, d_aux, (const float *)(w + B.dxe), dy, add_residual ? 1 : 0, (float *)(w + B.dh), dx,
                   dw_router, d_router_bias, (float *)(w + B.wpart), (float *)(w + B.bpart), w + B.aplanes,
                   w + B.bplanes, B.kp};
  if ((e = launch_router_bwd(ra, st, marks)) != hipSuccess) return hip_fail(e, "backward router launch");
  return SWITCH_OK;
}

// Between the two expert weight layouts (tile.hip); both directions share
// the checks.
int tile_call(int32_t count, int32_t rows, int32_t cols, const void *src, void *dst, void *stream,
              bool to_tiled) {
  if (count < 0 || rows < 0 || cols < 0)
    return fail(SWITCH_E_INVALID, "count = %d, rows = %d, cols = %d must be >= 0", count, rows, cols);
  if (rows % 16 || cols % 32)
    return fail(SWITCH_E_UNSUPPORTED, "rows = %d must be a multiple of 16 and cols = %d of 32", rows, cols);
  size_t bytes;
  if (!mul(bytes, {count, rows, cols, 2})) return fail(SWITCH_E_UNSUPPORTED, "matrix sizes overflow");
  if (bytes == 0) return SWITCH_OK;
  NEED(src, 16);
  NEED(dst, 16);
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
  if (a < b + bytes && b < a + bytes) return fail(SWITCH_E_INVALID, "src and dst overlap");
  TileArgs t{count, rows, cols, src, dst, to_tiled};
  return launched(launch_tile_weights(t, (hipStream_t)stream), to_tiled ? "tile launch" : "untile launch", stream);
}

// W_r [N][d] fp32 -> its three bf16 planes in the router's operand order.
int tile_router_bytes(int32_t num_experts, int32_t d_model, size_t &bytes) {
  if (num_experts < 1 || d_model < 1)
    return fail(SWITCH_E_INVALID, "num_experts = %d and d_model = %d must be >= 1", num_experts, d_model);
  if (d_model % 64) return fail(SWITCH_E_UNSUPPORTED, "d_model = %d must be a multiple of 64", d_model);
  size_t wr;
  if (!mul(wr, {num_experts, d_model, 4}) || !mul(bytes, {(num_experts + 15) / 16, d_model / 32, 3 * 64 * 16}))
    return fail(SWITCH_E_UNSUPPORTED, "sizes overflow");
  return SWITCH_OK;
}

int tile_router(int32_t num_experts, int32_t d_model, const float *w_router, void *planes, void *stream) {
  size_t bytes;
  int rc = tile_router_bytes(num_experts, d_model, bytes);
  if (rc) return rc;
  NEED(w_router, 16);
  NEED(planes, 16);
  const size_t wr = (size_t)num_experts * d_model * 4;
  const uintptr_t a = (uintptr_t)w_router, b = (uintptr_t)planes;
  if (a < b + bytes && b < a + wr) return fail(SWITCH_E_INVALID, "w_router and planes overlap");
  return launched(launch_router_planes(w_router, num_experts, d_model, planes, (hipStream_t)stream),
                  "tile_router launch", stream);
}

}  // namespace

extern "C" {

const char *switch_last_error(void) { return g_err.c_str(); }

int switch_capacity(int64_t tokens, int32_t num_experts, double cf, int32_t *capacity_out) {
  GUARD({
    if (!capacity_out) return fail(SWITCH_E_INVALID, "capacity_out is NULL");
    if (tokens < 0 || num_experts < 1 || !(cf > 0) || !std::isfinite(cf))
      return fail(SWITCH_E_INVALID, "need tokens >= 0, num_experts >= 1 and a finite capacity_factor > 0");
    if (tokens > INT32_MAX) return fail(SWITCH_E_UNSUPPORTED, "tokens above 2^31-1");
    if (tokens == 0) {
      *capacity_out = 0;
      return SWITCH_OK;
    }
    // cf = mant * 2^sh exactly; capacity = ceil(tokens * mant * 2^sh / N).
    int ex = 0;
    const double fr = std::frexp(cf, &ex);
    int64_t mant = (int64_t)std::ldexp(fr, 53);
    int sh = ex - 53;
    while ((mant & 1) == 0) {
      mant >>= 1;
      ++sh;
    }
    unsigned __int128 num = (unsigned __int128)tokens * (unsigned __int128)mant;  // < 2^84
    unsigned __int128 den = (unsigned __int128)num_experts;
    if (sh > 0) {
      if (sh > 40) return fail(SWITCH_E_UNSUPPORTED, "capacity above 2^31-1");
      num <<= sh;
    } else if (sh < 0) {
      if (-sh >= 90) {
        *capacity_out = 1;  // 0 < T*cf/N < 1
        return SWITCH_OK;
      }
      den <<= -sh;
    }
    unsigned __int128 q = num / den;
    if (q * den != num) ++q;
    if (q > (unsigned __int128)INT32_MAX) return fail(SWITCH_E_UNSUPPORTED, "capacity above 2^31-1");
    *capacity_out = (int32_t)q;
    return SWITCH_OK;
  })
}

int switch_workspace_bytes(const switch_shape *s, size_t *bytes_out) {
  GUARD({
    if (!bytes_out) return fail(SWITCH_E_INVALID, "bytes_out is NULL");
    int rc = check_shape(s);
    if (rc) return rc;
    Layout L;
    if ((rc = layout(s, L))) return rc;
    *bytes_out = L.total;
    return SWITCH_OK;
  })
}

int switch_route(const switch_shape *s, const void *x, const float *w_router, const float *router_bias,
                 int32_t *expert_idx, float *gate, int32_t *slot, uint8_t *dropped, int32_t *expert_count,
                 float *aux_loss, void *ws, size_t ws_bytes, void *stream) {
  GUARD({
    int rc = check_shape(s);
    if (rc) return rc;
    Layout L;
    if ((rc = layout(s, L))) return rc;
    RouteArgs a;
    if ((rc = route_args(s, x, w_router, router_bias, expert_idx, gate, slot, dropped, expert_count, aux_loss, ws,
                         ws_bytes, L, a)))
      return rc;
    Timer tm(stream);
    return tm.done(run_route(a, (hipStream_t)stream, tm));
  })
}

int switch_route_dispatch(const switch_shape *s, const void *x, const float *w_router, const float *router_bias,
                          int32_t *expert_idx, float *gate, int32_t *slot, uint8_t *dropped,
                          int32_t *expert_count, float *aux_loss, void *dispatched, void *ws, size_t ws_bytes,
                          void *stream) {
  GUARD({
    int rc = check_shape(s);
    if (rc) return rc;
    if (s->num_experts > kFusedMaxExperts)
      return fail(SWITCH_E_UNSUPPORTED, "num_experts = %d above %d", s->num_experts, kFusedMaxExperts);
    if ((int64_t)s->num_experts * s->capacity > INT32_MAX)
      return fail(SWITCH_E_UNSUPPORTED, "num_experts x capacity above 2^31-1");
    Layout L;
    if ((rc = layout(s, L))) return rc;
    FusedRouteArgs a;
    if ((rc = route_args(s, x, w_router, router_bias, expert_idx, gate, slot, dropped, expert_count, aux_loss, ws,
                         ws_bytes, L, a.r)))
      return rc;
    if (s->tokens > 0 && s->capacity > 0) NEED(dispatched, 16);
    char *w = (char *)ws;
    a.sync = (int32_t *)(w + L.fz_sync);
    a.clear_bytes = L.fz_clear;
    a.row_stride = L.fz_stride;
    a.agg_c = (int32_t *)(w + L.fz_aggc);
    a.inc_c = (int32_t *)(w + L.fz_incc);
    a.agg_p = (int64_t *)(w + L.fz_aggp);
    a.inc_p = (int64_t *)(w + L.fz_incp);
    a.dispatched = s->capacity > 0 ? dispatched : nullptr;
    Timer tm(stream);
    LaunchMarks marks{[](void *ctx, const char *name) { static_cast<Timer *>(ctx)->mark(name); },
                      [](void *ctx) { return static_cast<Timer *>(ctx)->reps(); }, &tm};
    hipError_t e = launch_route_fused(a, (hipStream_t)stream, marks);
    return tm.done(e == hipSuccess ? SWITCH_OK : hip_fail(e, "route_dispatch launch"));
  })
}

int switch_dispatch(const switch_shape *s, const void *x, const int32_t *expert_idx, const int32_t *slot,
                    const uint8_t *dropped, void *dispatched, void *stream) {
  GUARD({
    int rc = check_shape(s);
    if (rc) return rc;
    if (s->tokens > 0) {
      NEED(x, 16);
      NEED(expert_idx, 4);
      NEED(slot, 4);
      if (!dropped) return fail(SWITCH_E_INVALID, "dropped is NULL");
      if (s->capacity > 0) NEED(dispatched, 16);
    }
    DispatchArgs a{s->dtype, s->tokens, s->d_model, s->num_experts, s->capacity, x,
                   expert_idx, slot, dropped, dispatched};
    hipError_t e = launch_dispatch(a, (hipStream_t)stream);
    return launched(e, "dispatch launch", stream);
  })
}

int switch_expert_ffn(const switch_shape *s, const void *dispatched, const int32_t *expert_count,
                      const void *w_in, const void *w_out, void *expert_out, void *ws, size_t ws_bytes,
                      void *stream) {
  GUARD({
    int rc = check_shape(s);
    if (rc) return rc;
    Layout L;
    if ((rc = layout(s, L))) return rc;
    NEED(expert_count, 4);
    NEED(w_in, 16);
    NEED(w_out, 16);
    if (s->capacity > 0) {
      NEED(dispatched, 16);
      NEED(expert_out, 16);
    }
    if ((rc = check_ws(ws, ws_bytes, L.ffn_end))) return rc;
    FfnArgs a{s->dtype, s->d_model, s->d_ff, s->num_experts, s->capacity, dispatched, expert_count,
              w_in, w_out, (char *)ws + L.ffn_hidden, expert_out, tiled(s)};
    if ((rc = launched(launch_ffn_up(a, (hipStream_t)stream), "ffn_up launch", stream))) return rc;
    return launched(launch_ffn_down(a, (hipStream_t)stream), "ffn_down launch", stream);
  })
}

int switch_combine(const switch_shape *s, const void *expert_out, const int32_t *expert_idx, const int32_t *slot,
                   const uint8_t *dropped, const float *gate, const void *x_residual, void *y, void *stream) {
  GUARD({
    int rc = check_shape(s);
    if (rc) return rc;
    if (s->tokens > 0) {
      NEED(expert_idx, 4);
      NEED(slot, 4);
      NEED(gate, 4);
      NEED(y, 16);
      if (!dropped) return fail(SWITCH_E_INVALID, "dropped is NULL");
      if (s->capacity > 0) NEED(expert_out, 16);
      if (x_residual && !aligned(x_residual, 16))
        return fail(SWITCH_E_INVALID, "x_residual is not 16-byte aligned");
    }
    CombineArgs a{s->dtype, s->tokens, s->d_model, s->num_experts, s->capacity, expert_out,
                  expert_idx, slot, dropped, gate, x_residual, y};
    hipError_t e = launch_combine(a, (hipStream_t)stream);
    return launched(e, "combine launch", stream);
  })
}

int switch_add_norm(const switch_shape *s, const void *x, const void *y, const float *gamma, const float *beta,
                    float eps, void *out, void *stream) {
  GUARD({
    int rc = check_shape(s);
    if (rc) return rc;
    if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(SWITCH_E_INVALID, "eps = %g: need a finite eps >= 0", eps);
    if (s->d_model > add_norm_max_d(s->dtype))
      return fail(SWITCH_E_UNSUPPORTED, "d_model = %d above %d for add_norm", s->d_model,
                  add_norm_max_d(s->dtype));
    if (s->tokens > 0) {
      NEED(y, 16);
      NEED(out, 16);
      NEED(gamma, 4);
      NEED(beta, 4);
      if (x && !aligned(x, 16)) return fail(SWITCH_E_INVALID, "x is not 16-byte aligned");
    }
    AddNormArgs a{s->dtype, s->tokens, s->d_model, x, y, gamma, beta, eps, out, CombineRows{}};
    hipError_t e = launch_add_norm(a, (hipStream_t)stream);
    return launched(e, "add_norm launch", stream);
  })
}

int switch_combine_add_norm(const switch_shape *s, const void *expert_out, const int32_t *expert_idx,
                            const int32_t *slot, const uint8_t *dropped, const float *gate, const void *x,
                            const float *gamma, const float *beta, float eps, void *out, void *stream) {
  GUARD({
    int rc = check_shape(s);
    if (rc) return rc;
    if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(SWITCH_E_INVALID, "eps = %g: need a finite eps >= 0", eps);
    if (s->d_model > add_norm_max_d(s->dtype))
      return fail(SWITCH_E_UNSUPPORTED, "d_model = %d above %d for add_norm", s->d_model,
                  add_norm_max_d(s->dtype));
    if (s->tokens > 0) {
      NEED(x, 16);
      NEED(out, 16);
      NEED(expert_idx, 4);
      NEED(slot, 4);
      NEED(gate, 4);
      NEED(gamma, 4);
      NEED(beta, 4);
      if (!dropped) return fail(SWITCH_E_INVALID, "dropped is NULL");
      if (s->capacity > 0) NEED(expert_out, 16);
    }
    CombineRows rows{expert_idx, slot, dropped, gate, s->capacity};
    AddNormArgs a{s->dtype, s->tokens, s->d_model, x, expert_out, gamma, beta, eps, out, rows};
    hipError_t e = launch_add_norm(a, (hipStream_t)stream);
    return launched(e, "combine_add_norm launch", stream);
  })
}

int switch_layer_forward(const switch_shape *s, const void *x, const float *w_router, const float *router_bias,
                         const void *w_in, const void *w_out, int32_t add_residual, void *y, int32_t *expert_idx,
                         float *gate, int32_t *slot, uint8_t *dropped, int32_t *expert_count, float *aux_loss,
                         void *ws, size_t ws_bytes, void *stream) {
  GUARD({
    Timer tm(stream);
    return tm.done(layer_forward(s, 1, x, w_router, router_bias, w_in, w_out, add_residual, y, expert_idx, gate,
                                 slot, dropped, expert_count, aux_loss, ws, ws_bytes, stream, tm));
  })
}

int switch_layer_forward_train(const switch_shape *s, const void *x, const float *w_router,
                               const float *router_bias, const void *w_in, const void *w_out, int32_t add_residual,
                               void *y, int32_t *expert_idx, float *gate, int32_t *slot, uint8_t *dropped,
                               int32_t *expert_count, float *aux_loss, void *ws, size_t ws_bytes, void *stream) {
  GUARD({
    Timer tm(stream);
    return tm.done(layer_forward(s, 1, x, w_router, router_bias, w_in, w_out, add_residual, y, expert_idx, gate,
                                 slot, dropped, expert_count, aux_loss, ws, ws_bytes, stream, tm, true));
  })
}

int switch_layer_forward_add_norm(const switch_shape *s, const void *x, const float *w_router,
                                  const float *router_bias, const void *w_in, const void *w_out, const float *gamma,
                                  const float *beta, float eps, void *out, int32_t *expert_idx, float *gate,
                                  int32_t *slot, uint8_t *dropped, int32_t *expert_count, float *aux_loss, void *ws,
                                  size_t ws_bytes, void *stream) {
  GUARD({
    int rc = check_shape(s);
    if (rc) return rc;
    if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(SWITCH_E_INVALID, "eps = %g: need a finite eps >= 0", eps);
    if (s->d_model > add_norm_max_d(s->dtype))
      return fail(SWITCH_E_UNSUPPORTED, "d_model = %d above %d for the normalization", s->d_model,
                  add_norm_max_d(s->dtype));
    if (s->tokens > 0) {
      NEED(gamma, 4);
      NEED(beta, 4);
    }
    const NormOpt norm{gamma, beta, eps};
    Timer tm(stream);
    return tm.done(layer_forward(s, 1, x, w_router, router_bias, w_in, w_out, 0, out, expert_idx, gate, slot, dropped,
                                 expert_count, aux_loss, ws, ws_bytes, stream, tm, false, &norm));
  })
}

int switch_layer_forward_noalloc(const switch_shape *s, const void *x, const float *w_router,
                                 const float *router_bias, const void *w_in, const void *w_out, int32_t add_residual,
                                 void *y, int32_t *expert_idx, float *gate, int32_t *slot, uint8_t *dropped,
                                 int32_t *expert_count, float *aux_loss, void *stream) {
  GUARD({
    int rc = check_shape(s);
    if (rc) return rc;
    Layout L;
    if ((rc = layout(s, L))) return rc;
    if (L.total > kNoAllocScratchBytes)
      return fail(SWITCH_E_WORKSPACE, "this shape needs %zu bytes of workspace; the no-allocation call has %zu",
                  L.total, kNoAllocScratchBytes);
    void *ws = scratch_address();
    if (!ws) return SWITCH_E_HIP;
    Timer tm(stream);
    return tm.done(layer_forward(s, 1, x, w_router, router_bias, w_in, w_out, add_residual, y, expert_idx, gate,
                                 slot, dropped, expert_count, aux_loss, ws, kNoAllocScratchBytes, stream, tm));
  })
}

int switch_noalloc_scratch_bytes(size_t *bytes_out) {
  GUARD({
    if (!bytes_out) return fail(SWITCH_E_INVALID, "bytes_out is NULL");
    *bytes_out = kNoAllocScratchBytes;
    return SWITCH_OK;
  })
}

int switch_layer_forward_profiled(const switch_shape *s, const void *x, const float *w_router,
                                  const float *router_bias, const void *w_in, const void *w_out,
                                  int32_t add_residual, void *y, int32_t *expert_idx, float *gate, int32_t *slot,
                                  uint8_t *dropped, int32_t *expert_count, float *aux_loss, void *ws,
                                  size_t ws_bytes, void *stream, int32_t first_kernel, int32_t last_kernel,
                                  int32_t times) {
  GUARD({
    if (times < 1) return fail(SWITCH_E_INVALID, "times = %d < 1", times);
    if (first_kernel < 0 || last_kernel < first_kernel)
      return fail(SWITCH_E_INVALID, "kernel range %d..%d", first_kernel, last_kernel);
    Timer tm(stream);
    tm.first = first_kernel;
    tm.last = last_kernel;
    tm.times = times;
    int rc = tm.done(layer_forward(s, 1, x, w_router, router_bias, w_in, w_out, add_residual, y, expert_idx, gate,
                                   slot, dropped, expert_count, aux_loss, ws, ws_bytes, stream, tm));
    if (rc == SWITCH_OK && last_kernel >= tm.n)
      return fail(SWITCH_E_INVALID, "kernel range %d..%d: the call launches %d kernels", first_kernel, last_kernel,
                  tm.n);
    return rc;
  })
}

int switch_topk_workspace_bytes(const switch_shape *s, int32_t top_k, size_t *bytes_out) {
  GUARD({
    if (!bytes_out) return fail(SWITCH_E_INVALID, "bytes_out is NULL");
    int rc = check_shape(s);
    if (rc) return rc;
    if ((rc = check_topk(s, top_k))) return rc;
    Layout L;
    if ((rc = layout(s, L, top_k))) return rc;
    *bytes_out = L.total;
    return SWITCH_OK;
  })
}

int switch_topk_layer_forward(const switch_shape *s, int32_t top_k, const void *x, const float *w_router,
                              const float *router_bias, const void *w_in, const void *w_out, int32_t add_residual,
                              void *y, int32_t *expert_idx, float *gate, int32_t *slot, uint8_t *dropped,
                              int32_t *expert_count, float *aux_loss, void *ws, size_t ws_bytes, void *stream) {
  GUARD({
    Timer tm(stream);
    return tm.done(layer_forward(s, top_k, x, w_router, router_bias, w_in, w_out, add_residual, y, expert_idx, gate,
                                 slot, dropped, expert_count, aux_loss, ws, ws_bytes, stream, tm));
  })
}

int switch_backward_workspace_bytes(const switch_shape *s, size_t *bytes_out) {
  GUARD({
    if (!bytes_out) return fail(SWITCH_E_INVALID, "bytes_out is NULL");
    int rc = check_shape(s);
    if (rc) return rc;
    BwdLayout B;
    if ((rc = bwd_layout(s, B))) return rc;
    *bytes_out = B.total;
    return SWITCH_OK;
  })
}

int switch_layer_backward(const switch_shape *s, const void *x, const float *w_router, const float *router_bias,
                          const void *w_in, const void *w_out, int32_t add_residual, const int32_t *expert_idx,
                          const uint8_t *dropped, const int32_t *expert_count, const void *fwd_workspace,
                          size_t fwd_workspace_bytes, const void *dy, float d_aux, void *dx, float *dw_router,
                          float *d_router_bias, void *dw_in, void *dw_out, void *workspace, size_t workspace_bytes,
                          void *stream) {
  GUARD({
    Timer tm(stream);
    return tm.done(layer_backward(s, x, w_router, router_bias, w_in, w_out, add_residual, expert_idx, dropped,
                                  expert_count, fwd_workspace, fwd_workspace_bytes, dy, d_aux, dx, dw_router,
                                  d_router_bias, dw_in, dw_out, workspace, workspace_bytes, stream, tm));
  })
}

int switch_layer_backward_profiled(const switch_shape *s, const void *x, const float *w_router,
                                   const float *router_bias, const void *w_in, const void *w_out,
                                   int32_t add_residual, const int32_t *expert_idx, const uint8_t *dropped,
                                   const int32_t *expert_count, const void *fwd_workspace,
                                   size_t fwd_workspace_bytes, const void *dy, float d_aux, void *dx,
                                   float *dw_router, float *d_router_bias, void *dw_in, void *dw_out,
                                   void *workspace, size_t workspace_bytes, void *stream, int32_t first_kernel,
                                   int32_t last_kernel, int32_t times) {
  GUARD({
    if (times < 1) return fail(SWITCH_E_INVALID, "times = %d < 1", times);
    if (first_kernel < 0 || last_kernel < first_kernel)
      return fail(SWITCH_E_INVALID, "kernel range %d..%d", first_kernel, last_kernel);
    Timer tm(stream);
    tm.first = first_kernel;
    tm.last = last_kernel;
    tm.times = times;
    int rc = tm.done(layer_backward(s, x, w_router, router_bias, w_in, w_out, add_residual, expert_idx, dropped,
                                    expert_count, fwd_workspace, fwd_workspace_bytes, dy, d_aux, dx, dw_router,
                                    d_router_bias, dw_in, dw_out, workspace, workspace_bytes, stream, tm));
    if (rc == SWITCH_OK && last_kernel >= tm.n)
      return fail(SWITCH_E_INVALID, "kernel range %d..%d: the call launches %d kernels", first_kernel, last_kernel,
                  tm.n);
    return rc;
  })
}

int switch_tile_weights(int32_t count, int32_t rows, int32_t cols, const void *src, void *dst, void *stream) {
  GUARD({ return tile_call(count, rows, cols, src, dst, stream, true); })
}

int switch_untile_weights(int32_t count, int32_t rows, int32_t cols, const void *src, void *dst, void *stream) {
  GUARD({ return tile_call(count, rows, cols, src, dst, stream, false); })
}

int switch_tiled_router_bytes(int32_t num_experts, int32_t d_model, size_t *bytes_out) {
  GUARD({
    if (!bytes_out) return fail(SWITCH_E_INVALID, "bytes_out is NULL");
    return tile_router_bytes(num_experts, d_model, *bytes_out);
  })
}

int switch_tile_router(int32_t num_experts, int32_t d_model, const float *w_router, void *planes, void *stream) {
  GUARD({ return tile_router(num_experts, d_model, w_router, planes, stream); })
}

int switch_launch_names(const switch_shape *s, const char **names, int32_t max_names, int32_t *num_names) {
  GUARD({
    if (!num_names || max_names < 0 || (max_names > 0 && !names))
      return fail(SWITCH_E_INVALID, "names / num_names is NULL or max_names < 0");
    int rc = check_shape(s);
    if (rc) return rc;
    const char *seq[kNumKernels];
    int n = 0;
    seq[n++] = "router";
    if (s->tokens == 0 || assign_single_launch(router_blocks(s->tokens), s->num_experts)) {
      seq[n++] = "assign";
    } else {
      seq[n++] = "assign_scan";
      seq[n++] = "assign_apply";
    }
    if (fused_ffn(s, false)) {
      seq[n++] = "ffn";
    } else {
      seq[n++] = "ffn_up";
      seq[n++] = "ffn_down";
    }
    for (int i = 0; i < n && i < max_names; ++i) names[i] = seq[i];
    *num_names = n;
    return SWITCH_OK;
  })
}

}  // extern "C"
