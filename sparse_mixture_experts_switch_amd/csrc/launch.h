// Internal launch interface between the C ABI (abi.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace smx {

enum Dtype { kF32 = 0, kBF16 = 1 };

constexpr int kRouterTokens = 64;    // tokens per router block
constexpr int kRouterThreads = 256;  // 4 waves
constexpr int kRouterChunk = 128;    // experts per logits chunk (4 waves x 32)

// Routing arguments.  k routes per token (1: Switch routing; 2: classic
// top-2).  Route r of token t is "virtual token" r * Tp + t with Tp =
// router_blocks(T) * kRouterTokens, so the router block b of route r is block
// r * nb + b of the assignment; per-route outputs (expert_idx, gate, slot,
// dropped) are [k][T].
struct RouteArgs {
  int dtype;
  int k;
  int64_t T;
  int d, N, C;
  const void *x;
  const float *w_r, *bias;
  float *logits;  // [T][N] scratch, only used when N > kRouterChunk
  void *wplanes;  // bf16 layers: W_r split into bf16 planes in MFMA fragment order (router_planes_bytes)
  bool wr_planes = false;  // wplanes is the caller's W_r already in that form (tiled weights): no split pass
  int32_t *expert_idx;
  float *gate;
  int32_t *slot;  // slot of each token (assignment output)
  int32_t *rank;  // [k * Tp] workspace: rank of each route among its block's earlier routes to the same expert
  uint8_t *dropped;
  int32_t *expert_count;
  float *aux_loss;
  int32_t *bcount;  // [k * nb][count_stride(N)]: block counts
  int32_t *boff;    // [k * nb][count_stride(N)]: exclusive block offsets (scan path)
  float *ppart;     // [k * nb][count_stride(N)]: block partial sums of p (route 0 rows; others 0)
  float *psum;      // [N]
};

struct DispatchArgs {
  int dtype;
  int64_t T;
  int d, N, C;
  const void *x;
  const int32_t *expert_idx, *slot;
  const uint8_t *dropped;
  void *dispatched;  // [N][C][d]
};

struct FfnArgs {
  int dtype;
  int d, dff, N, C;
  const void *dispatched;  // [N][C][d]
  const int32_t *expert_count;
  const void *w_in;   // [N][dff][d]
  const void *w_out;  // [N][d][dff]
  void *hidden;       // [N][C][dff] scratch
  void *expert_out;   // [N][C][d]
  bool tiled = false; // weights in MFMA operand order (bf16), see tile_weights
};

struct CombineArgs {
  int dtype;
  int64_t T;
  int d, N, C;
  const void *expert_out;
  const int32_t *expert_idx, *slot;
  const uint8_t *dropped;
  const float *gate;
  const void *x_residual;  // may be null
  void *y;
};

// Rows of the stage API's combine (gate * expert_out[e][slot], 0 if dropped).
struct CombineRows {
  const int32_t *expert_idx = nullptr, *slot = nullptr;
  const uint8_t *dropped = nullptr;
  const float *gate = nullptr;
  int C = 0;
};

struct AddNormArgs {
  int dtype;
  int64_t T;
  int d;
  const void *x;  // may be null
  const void *y;  // [T][d], or expert_out [N][C][d] when rows.expert_idx is set
  const float *gamma, *beta;
  float eps;
  void *out;  // may equal y (dense rows only)
  CombineRows rows;
};

// One grouped GEMM of the expert FFN (see ffn.hip).
struct GemmCall {
  int dtype, N, C, K, Nout;
  const void *A;  // [N][C][K] buffer, or x [T][K] when rows are gathered through tok
  const void *B;  // [N][Nout][K]
  void *Out;      // [N][C][Nout] buffer, or y [T][Nout] for the combine epilogue
  const int32_t *counts;
  const int32_t *tok;  // [N][C]: token in each live slot (gather / combine)
  const float *gate;   // [T] (combine, fp32 path)
  const float *gmap;   // [N][C]: gate of the token in each live slot (combine)
  const void *xres;    // [T][Nout] residual rows (combine), may be null
  bool tiled = false;  // B in MFMA operand order (bf16), see tile_weights
  int64_t out_rows = 0;  // combine: rows of y (its size decides the store policy)
};

// Compute units of the current device, queried once per device (256 when the
// query fails); the launchers size persistent grids with it.
constexpr int kMaxDeviceCache = 64;
int device_cus();

// Each launcher enqueues its kernels on `st` and returns the launch status.
hipError_t launch_router(const RouteArgs &a, hipStream_t st);
// Capacity assignment and loss after the router.  Small batches take one
// launch (each workgroup sums the counts of the blocks before its own);
// others a scan over blocks, then the apply step.  With tok set (layer path)
// it also records, for each kept route of token t, tok[e][slot] = t, the
// route's output row rows[e][slot] = r * T + t (rows may be null when k = 1:
// the row is t) and its gate gmap[e][slot], and, when y is set (k = 1 only),
// writes the y rows of dropped tokens (0, or x with a residual).
// marks.fn (may be null) is called with each kernel's name after its
// launches; marks.reps (may be null) says how many times to issue the next
// kernel back to back (measurement only: no kernel modifies its inputs).
struct LaunchMarks {
  void (*fn)(void *ctx, const char *name);
  int (*reps)(void *ctx);
  void *ctx;
};
// Whether the assignment of nb router blocks and N experts takes one launch.
bool assign_single_launch(int64_t nb, int N);
struct LayerMaps {
  int32_t *tok = nullptr;   // [N][C] token of each live slot (x row to gather)
  int32_t *rows = nullptr;  // [N][C] output row of each live slot, or null (= tok)
  float *gmap = nullptr;    // [N][C] gate of each live slot
  const void *xres = nullptr;
  void *y = nullptr;
  // with gamma set (and xres = x), the rows of dropped tokens are the block's
  // Add + Normalize of x alone: (x - mean) / sqrt(var + eps) * gamma + beta
  const float *gamma = nullptr, *beta = nullptr;
  float eps = 0.f;
};
hipError_t launch_assign(const RouteArgs &a, const LayerMaps &m, hipStream_t st, LaunchMarks marks);

// Single-pass routing with one route per token: the router kernel also
// assigns the capacity slots (each block adds the counts of the blocks before
// it, found by a look-back in token order), forms the totals and the loss,
// and, with dispatched set, copies each kept token's row of x to
// dispatched[e][slot].  r.bcount / r.ppart receive the block counts and P
// sums; r.logits is used as for launch_router.  A small kernel clears the
// first clear_bytes at `sync` (ticket, error word, block states) first; the
// two launches count as one step for LaunchMarks.
constexpr int kFusedMaxExperts = 2048;
struct FusedRouteArgs {
  RouteArgs r;
  int32_t *sync;          // [4 + nb]: block ticket, error word, 2 unused, then one state per block
  size_t clear_bytes;     // (4 + nb) * 4 rounded up to 16
  int64_t row_stride;     // of the rows below: N rounded up to 64
  int32_t *agg_c, *inc_c; // [nb][row_stride] block counts, counts of blocks 0..b
  int64_t *agg_p, *inc_p; // [nb][row_stride] P sums (2^-31 fixed point), the same
  void *dispatched;       // [N][C][d], or null
};
hipError_t launch_route_fused(const FusedRouteArgs &a, hipStream_t st, LaunchMarks marks);
// Top-k combine: y[t] = sum over kept routes r of routed[r * T + t] (+ x[t]).
struct TopkSumArgs {
  int dtype, k;
  int64_t T;
  int d;
  const void *routed;  // [k][T][d]
  const uint8_t *dropped;  // [k][T]
  const void *x;  // may be null
  void *y;
};
hipError_t launch_topk_sum(const TopkSumArgs &a, hipStream_t st);
// Expert weights [count][rows][cols] bf16 between row-major and the tiled
// layout (to_tiled) or back: element (r, c) of matrix m sits at
//   ((m (rows/16) + r/16) (cols/32) + c/32) 512 + (16 ((c % 32)/8) + r % 16) 8 + c % 8.
// rows % 16 == 0, cols % 32 == 0; src and dst do not overlap.
struct TileArgs {
  int64_t count;
  int rows, cols;
  const void *src;
  void *dst;
  bool to_tiled;
};
hipError_t launch_tile_weights(const TileArgs &a, hipStream_t st);
hipError_t launch_dispatch(const DispatchArgs &a, hipStream_t st);
hipError_t launch_ffn_up(const FfnArgs &a, hipStream_t st);
hipError_t launch_ffn_down(const FfnArgs &a, hipStream_t st);
hipError_t launch_ffn_up_gather(const GemmCall &c, hipStream_t st);
// Expert FFN and combine in one kernel (ffn_fused.hip): the hidden
// activations stay on chip.  Taken by the layer call when
// ffn_fused_eligible(dtype, d, d_ff, C).
struct FusedFfnCall {
  int dtype, N, C, d, dff;
  const void *x;           // [T][d]
  const void *w_in;        // [N][dff][d]
  const void *w_out;       // [N][d][dff]
  void *out;               // y [T][d], or the routed rows [k][T][d]
  const int32_t *counts;
  const int32_t *tok;      // [N][C]
  const int32_t *rows;     // [N][C] output row of each live slot, or null (= tok)
  const float *gmap;       // [N][C]
  const void *xres;        // residual rows, or null
  // set (k = 1, xres = x): write the block's Add + Normalize of x + y instead of y
  const float *gamma = nullptr, *beta = nullptr;
  float eps = 0.f;
  bool tiled = false;      // w_in / w_out in MFMA operand order, see tile_weights
};
bool ffn_fused_eligible(int dtype, int d, int dff, int C);
hipError_t launch_ffn_fused(const FusedFfnCall &c, hipStream_t st);
hipError_t launch_ffn_down_combine(const GemmCall &c, hipStream_t st);
hipError_t launch_combine(const CombineArgs &a, hipStream_t st);
hipError_t launch_add_norm(const AddNormArgs &a, hipStream_t st);
int add_norm_max_d(int dtype);  // largest d_model the row-in-registers kernel takes

// ---- backward pass ----
// Expert products of the backward (backward.hip), all on the forward's saved
// slot maps and hidden activations.
struct BwdLaunch {
  int dtype;
  int64_t T;
  int d, dff, N, C;
  const void *x, *w_in, *w_out, *dy;
  const int32_t *counts;  // expert_count from the forward
  const int32_t *tok;     // [N][C] slot -> token (forward workspace)
  const float *gmap;      // [N][C] slot -> gate (forward workspace)
  const void *hidden;     // [N][C][dff] H (forward workspace)
  void *du;               // [N][C][dff] out: g z [H > 0]
  float *dgpart;          // [T][bwd_dz_tiles] out: partial <z, H> per token
  float *dxe;             // [T][d] out: W_in^T du for kept tokens (fp32)
  void *dw_in, *dw_out;   // out: weight gradients, activation dtype
};
int bwd_dz_tiles(int dtype, int dff);
hipError_t launch_bwd_experts(const BwdLaunch &a, hipStream_t st, LaunchMarks marks);

// Router part of the backward (router.hip): recomputes the logits, forms
// dL/dh (softmax Jacobian of dL/dp = d_aux N f / T + [kept, chosen] dL/dg),
// writes dh and the bias partials, and the whole dx (fp32 layers: in the
// same kernel; bf16 layers: the exact bf16 planes of dL/dh, then the MFMA dx
// product of backward.hip); then dW_r by a split sum over tokens and the
// ordered sums of the partials.
struct RouterBwdArgs {
  int dtype;
  int64_t T;
  int d, N;
  const void *x;
  const float *w_r, *bias;
  float *logits;  // [T][N] scratch when N > kRouterChunk
  void *wplanes;  // bf16 layers: router_planes_bytes of scratch for the logits' W_r planes
  const int32_t *expert_idx;
  const uint8_t *dropped;
  const int32_t *expert_count;
  const float *dgpart;  // [T][n_dg]
  int n_dg;
  float d_aux;
  const float *dxe;  // [T][d]
  const void *dy;
  int add_residual;
  float *dh;  // [T][N] out
  void *dx;   // [T][d] out
  float *dw_r, *dbias;    // out ([N][d], [N] or null)
  float *wpart;           // [splits][N][d] scratch: dW_r partial sums
  float *bpart;           // [router blocks][N] scratch: bias partial sums
  void *aplanes;          // bf16 layers: [T][kp] dL/dh planes for the dx product
  void *bplanes;          // bf16 layers: [kp][d] W_r planes
  int kp;
};
// The router's part of dx on bf16 MFMA (backward.hip), with the experts' part
// and dy added: the whole dx of a bf16 layer.
struct RouterDxArgs {
  int64_t T;
  int d, N, kp;
  const float *w_r;
  const void *aplanes;
  void *bplanes;
  const float *dxe;
  const uint8_t *dropped;
  const void *dyres;  // dy with the residual, or null
  void *dx;
};
int router_dx_kp(int N);  // contraction length of the plane products, padded
hipError_t launch_router_dx_bf16(const RouterDxArgs &r, hipStream_t st);
// Token split of the dW_r sum: `splits` ranges of `ts` tokens (a multiple of 64).
struct WgradSplit {
  int splits;
  int64_t ts;
};
WgradSplit router_wgrad_split(int64_t T, int N, int d);
hipError_t launch_router_bwd(const RouterBwdArgs &a, hipStream_t st, LaunchMarks marks);
// dW_r partial sums on bf16 MFMA (backward.hip): dh split exactly into three
// bf16 planes, x bf16, so every product is exact and accumulates in fp32.
hipError_t launch_router_wgrad_bf16(const float *dh, const void *x, int64_t T, int N, int d, WgradSplit sp,
                                    float *wpart, hipStream_t st);

__host__ __device__ inline int64_t router_blocks(int64_t T) { return (T + kRouterTokens - 1) / kRouterTokens; }
// Bytes of W_r split into three bf16 planes, laid out in the order the bf16
// router's MFMA waves load them: [ceil(N / 16)][d / 32][3 planes][64 lanes]
// pieces of 16 bytes (written by a split pass before the router of each
// call, or once by the caller for tiled weights).
__host__ __device__ inline int64_t router_planes_bytes(int N, int d) {
  return (int64_t)((N + 15) / 16) * (d / 32) * 3 * 64 * 16;
}
// Writes those planes of W_r [N][d] fp32 (zeros for the experts past N in the
// last 16-expert tile).
hipError_t launch_router_planes(const float *w_r, int N, int d, void *wplanes, hipStream_t st);
// Row stride (elements) of the per-block count and P-partial arrays: rows
// start on 16-byte boundaries.
__host__ __device__ inline int count_stride(int N) { return (N + 3) & ~3; }

}  // namespace smx
