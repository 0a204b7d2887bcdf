// Router of the Switch layer: logits h = W_r . x (+ b), fp32 softmax, top-1
// expert, gate p_e(x), and the per-block partial results that the capacity
// assignment and the load-balancing loss are built from.  The same kernels
// also route each token to its two best experts (classic top-2 routing, the
// variant the Switch layer simplifies), with the gate p_i(x) of each.
//
// Switch Transformers write-up, "Switch Routing: From Top-k to k = 1" (router
// logits and the softmax gate equation), "Making Sparse Training Stable"
// (selective precision: the router works in fp32 on its fp32-cast input),
// "The Load-Balancing Loss" (P_i = mean router probability).
//
// One workgroup owns kRouterTokens consecutive tokens (one "router block").
// It computes their logits for every expert, chunk by chunk of up to
// kRouterChunk experts, and keeps them in LDS (or, for more experts than fit,
// in a global fp32 scratch row per token).  The epilogue then, per token:
// max and first argmax of the logits, s = sum_j exp(h_j - max), gate = 1/s;
// per block: P partial sums sum_t p_j(t) in token order, the number of the
// block's tokens that chose each expert, and each token's rank among the
// block's earlier tokens with the same expert (stored in rank[] and later
// offset by the cross-block scan).
//
// bf16 activations: the contraction runs on bf16 MFMA.  W_r (fp32) is split
// exactly into three bf16 planes hi + mid + lo (each plane takes the next 8
// significant bits), once per call by a small kernel that also lays them out
// in MFMA fragment order, so every product x_k * plane_k is exact in fp32 and
// the fp32 accumulation sees the same terms as an fp32 dot product.  The
// softmax uses the accurate expf (not the fast exp intrinsic) and an IEEE
// division for the gate.
// fp32 activations: plain fp32 FMA on the vector ALUs.

#include <algorithm>
#include <climits>

#include "common.h"
#include "launch.h"

namespace smx {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Exact split of two fp32 values into three bf16 pairs whose sums are the
// values: hi = bf16(w), mid = bf16(w - hi), lo = bf16(w - hi - mid), each
// conversion rounding to nearest even (both differences are exact in fp32).
// Each result holds the pair packed as two bf16 (first value in the low half).
__device__ __forceinline__ void split3_pair(f32x2 w, uint32_t &hi, uint32_t &mid, uint32_t &lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(w, bf16x2));
  const f32x2 r1 = w - f32x2{__builtin_bit_cast(float, hi << 16), __builtin_bit_cast(float, hi & 0xffff0000u)};
  mid = __builtin_bit_cast(uint32_t, __builtin_convertvector(r1, bf16x2));
  const f32x2 r2 = r1 - f32x2{__builtin_bit_cast(float, mid << 16), __builtin_bit_cast(float, mid & 0xffff0000u)};
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r2, bf16x2));
}

// The three bf16x8 planes of 8 consecutive fp32 values.
__device__ __forceinline__ void split3_x8(const f32x4 a, const f32x4 b, bf16x8 &hi, bf16x8 &mid, bf16x8 &lo) {
  uint32_t h[4], m[4], l[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    split3_pair(f32x2{a[2 * i], a[2 * i + 1]}, h[i], m[i], l[i]);
    split3_pair(f32x2{b[2 * i], b[2 * i + 1]}, h[2 + i], m[2 + i], l[2 + i]);
  }
  hi = as_bf16x8(u32x4{h[0], h[1], h[2], h[3]});
  mid = as_bf16x8(u32x4{m[0], m[1], m[2], m[3]});
  lo = as_bf16x8(u32x4{l[0], l[1], l[2], l[3]});
}

template <bool kLds>
struct LogitRows {
  float *base;      // LDS [kRouterTokens][stride] or global [T][N] (row t0)
  int64_t stride;
  __device__ __forceinline__ float &at(int t, int j) const { return base[(int64_t)t * stride + j]; }
};

// Softmax, top-k choice (k = 1 or 2), gates, P partials, block counts and
// in-block ranks for the block's tokens, from logits already complete in `lg`
// (kThreads threads).
//  - kThreads / 64 consecutive lanes share a token: each scans a strided
//    subset of the experts, butterfly steps combine the partial results in a
//    fixed order; exp(h_j - max) replaces h_j in `lg` on the way.  The order
//    of the choice is larger logit first, lower expert index first on equal
//    logits; it is a total order, so the butterfly partners agree exactly.
//  - kThreads / 128 consecutive lanes share an expert: each sums p_j(t) and
//    counts the choices of one contiguous run of the block's tokens, and the
//    runs are combined by butterfly steps (fixed order: the same bits every
//    call).
// Route r of token t0 + t is written at r * T + t0 + t (expert_idx, gate) and
// r * Tp + t0 + t (rank, Tp = nb * kRouterTokens); its block counts are row
// r * nb + blk of bcount.  The P partials go to row blk; rows nb + blk of a
// second route hold zeros (P does not depend on the route).
struct TopK {
  int64_t T, nb;  // tokens, router blocks
};

// A block's P partial sum (fp32, at most 64) in 2^-31 fixed point: exact for
// sums of at least 2^-8, rounded to nearest below.  Integer sums of these are
// independent of their order, so totals formed in any grouping agree bit for
// bit.
__device__ __forceinline__ int64_t p_fixed(float p) { return __double2ll_rn((double)p * 0x1p31); }

// The best (and second best) logit of a lane and its expert.  Every update
// is a select of values: conditional assignments through the references made
// the compiler keep the four values of the top-2 epilogue in scratch memory
// (a dependent chain of scratch accesses per logit).
template <int kK>
__device__ __forceinline__ void topk_take(float h, int j, float &b1, int &i1, float &b2, int &i2) {
  // ascending j within one lane: strict comparisons keep the lower index
  const bool g1 = h > b1;
  if (kK == 2) {
    const bool g2 = h > b2;
    const float nb2 = g1 ? b1 : (g2 ? h : b2);
    const int ni2 = g1 ? i1 : (g2 ? j : i2);
    b2 = nb2;
    i2 = ni2;
  }
  b1 = g1 ? h : b1;
  i1 = g1 ? j : i1;
}

__device__ __forceinline__ bool topk_before(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// Merge another lane's ordered (best, second) into this lane's: the top two
// of the union (larger logit first, the lower index on equal logits).
template <int kK>
__device__ __forceinline__ void topk_merge(float ov, int oi, float ov2, int oi2, float &best, int &bi, float &sec,
                                           int &si) {
  const bool theirs = topk_before(ov, oi, best, bi);
  if (kK == 2) {
    const bool mine2 = topk_before(best, bi, ov2, oi2);  // theirs first: second is my first or their second
    const bool osec = topk_before(ov, oi, sec, si);      // mine first: second is their first or my second
    const float ns = theirs ? (mine2 ? best : ov2) : (osec ? ov : sec);
    const int nsi = theirs ? (mine2 ? bi : oi2) : (osec ? oi : si);
    sec = ns;
    si = nsi;
  }
  best = theirs ? ov : best;
  bi = theirs ? oi : bi;
}

// With s_cnt set (one route per token) the block's counts and P partial sums
// also go to LDS, the sums as 2^-31 fixed point (s_pfix), for the single-pass
// assignment that follows in the same kernel.
template <int kThreads, bool kLds, int kK>
__device__ __forceinline__ void router_epilogue(const LogitRows<kLds> lg, int nt, int N, int64_t t0, int64_t blk, TopK tk,
                                int32_t *__restrict__ expert_idx, float *__restrict__ gate,
                                int32_t *__restrict__ slot_rank, int32_t *__restrict__ bcount,
                                float *__restrict__ ppart, float *s_max, float *s_inv, int *s_e, int *s_e2,
                                int *s_cnt = nullptr, int64_t *s_pfix = nullptr) {
  constexpr int kLpt = kThreads / kRouterTokens;   // lanes per token
  constexpr int kTpe = kThreads / kRouterChunk;    // lanes per expert
  constexpr int kUpt = kRouterTokens / kTpe;       // tokens per lane in the expert sums
  static_assert(kLpt >= 1 && kLpt <= kWave && (kLpt & (kLpt - 1)) == 0, "lanes per token");
  static_assert(kTpe >= 1 && kTpe <= kWave && (kTpe & (kTpe - 1)) == 0, "lanes per expert");
  static_assert(kK == 1 || kK == 2, "one or two routes per token");
  const int tid = threadIdx.x;
  const int t = tid / kLpt, q = tid % kLpt;
  if (t < nt) {  // the lanes of a token are always on the same side of t < nt
    float best = -INFINITY, sec = -INFINITY;
    int bi = 0x7fffffff, si = 0x7fffffff;
    if (kLds) {  // N <= kRouterChunk: at most kJ values per lane, loaded together
      constexpr int kJ = kRouterChunk / kLpt;
      float h[kJ];
#pragma unroll
      for (int i = 0; i < kJ; ++i) h[i] = q + i * kLpt < N ? lg.at(t, q + i * kLpt) : -INFINITY;
#pragma unroll
      for (int i = 0; i < kJ; ++i)
        if (q + i * kLpt < N) topk_take<kK>(h[i], q + i * kLpt, best, bi, sec, si);
    } else {
      for (int j = q; j < N; j += kLpt) topk_take<kK>(lg.at(t, j), j, best, bi, sec, si);
    }
#pragma unroll
    for (int off = 1; off < kLpt; off <<= 1) {
      const float ov = __shfl_xor(best, off, kWave);
      const int oi = __shfl_xor(bi, off, kWave);
      const float ov2 = kK == 2 ? __shfl_xor(sec, off, kWave) : 0.f;
      const int oi2 = kK == 2 ? __shfl_xor(si, off, kWave) : 0;
      topk_merge<kK>(ov, oi, ov2, oi2, best, bi, sec, si);
    }
    float sum = 0.f;
    if (kLds) {
      constexpr int kJ = kRouterChunk / kLpt;
      float ev[kJ];
#pragma unroll
      for (int i = 0; i < kJ; ++i) ev[i] = q + i * kLpt < N ? expf(lg.at(t, q + i * kLpt) - best) : 0.f;
#pragma unroll
      for (int i = 0; i < kJ; ++i) {
        if (q + i * kLpt < N) lg.at(t, q + i * kLpt) = ev[i];
        sum += ev[i];
      }
    } else {
      for (int j = q; j < N; j += kLpt) {
        const float ev = expf(lg.at(t, j) - best);
        lg.at(t, j) = ev;
        sum += ev;
      }
    }
#pragma unroll
    for (int off = 1; off < kLpt; off <<= 1) sum += __shfl_xor(sum, off, kWave);
    if (q == 0) {
      const float inv = 1.0f / sum;
      s_max[t] = best;
      s_inv[t] = inv;
      s_e[t] = bi;
      expert_idx[t0 + t] = bi;
      gate[t0 + t] = inv;  // p_e = exp(h_e - max) / sum with h_e = max
      if (kK == 2) {
        s_e2[t] = si;
        expert_idx[tk.T + t0 + t] = si;
        gate[tk.T + t0 + t] = expf(sec - best) * inv;
      }
    }
  }
  __syncthreads();
  const int64_t Np = count_stride(N);
  for (int j0 = 0; j0 < N; j0 += kRouterChunk) {
    const int j = j0 + tid / kTpe, r = tid % kTpe;
    float p = 0.f;
    int c = 0, c2 = 0;
    if (j < N && tid < kThreads) {
#pragma unroll
      for (int i = 0; i < kUpt; ++i) {
        const int u = r * kUpt + i;
        if (u < nt) {
          p += lg.at(u, j) * s_inv[u];
          c += (s_e[u] == j);
          if (kK == 2) c2 += (s_e2[u] == j);
        }
      }
    }
#pragma unroll
    for (int off = 1; off < kTpe; off <<= 1) {
      p += __shfl_xor(p, off, kWave);
      c += __shfl_xor(c, off, kWave);
      if (kK == 2) c2 += __shfl_xor(c2, off, kWave);
    }
    if (r == 0 && j < N && tid < kThreads) {
      ppart[blk * Np + j] = p;
      bcount[blk * Np + j] = c;
      if (kK == 1 && s_cnt) {
        s_cnt[j] = c;
        s_pfix[j] = p_fixed(p);
      }
      if (kK == 2) {
        ppart[(tk.nb + blk) * Np + j] = 0.f;
        bcount[(tk.nb + blk) * Np + j] = c2;
      }
    }
  }
  // rank among the block's earlier tokens with the same expert, per route:
  // wave 0 holds one token per lane and reads the others' choices lane by lane
  static_assert(kRouterTokens == kWave, "one router block = one wave of tokens");
  if (tid < kWave) {
#pragma unroll 1
    for (int rt = 0; rt < kK; ++rt) {
      const int e = tid < nt ? (rt == 0 ? s_e[tid] : s_e2[tid]) : -1;
      int r = 0;
#pragma unroll
      for (int u = 0; u < kWave; ++u) r += (u < tid) & (__builtin_amdgcn_readlane(e, u) == e);
      if (tid < nt) slot_rank[rt * tk.nb * kRouterTokens + t0 + tid] = r;
    }
  }
}

// Threads of the router epilogue (8 waves: 8 lanes per token, 4 per expert),
// 16-token MFMA tiles per router block, and the LDS logit rows of a block
// when every expert fits one chunk: 160 floats per token (a row starts 32
// banks after the previous one, so the epilogue's 16-byte row reads and its
// column reads are free of bank conflicts).
constexpr int kRBThreads = 512;
constexpr int kTokTiles = kRouterTokens / 16;
constexpr int kLgStride = 160;
constexpr int kRouterLgBytes = kRouterTokens * kLgStride * 4;

// ---------------------------------------------------------------------------
// Forward router, bf16 activations: the layer's routing step.  Each
// workgroup owns one router block (64 tokens) and runs 12 waves in two roles:
//  - waves 8..11 stream the block's rows of x through LDS in chunks of 256
//    contraction columns (double-buffered: chunk 0 is requested alone so
//    that it arrives first, then each thread keeps the next two chunks in
//    registers);
//  - waves 0..7 multiply: wave w owns experts [c0 + 16 w, c0 + 16 w + 16) of
//    a 128-expert chunk for all 64 tokens (with at most 4 or 2 live expert
//    tiles, the waves share a tile and split the 64 tokens instead).  Its
//    operands of W_r's three exact bf16 planes (hi, mid, lo; fragment order,
//    see router_wplanes_kernel) come straight from global memory (590 KB,
//    held in every XCD's L2) into registers, three 1 KB pieces per wave and
//    32-column step, four steps ahead; the x operands are 16-byte LDS reads.
//    Each plane has its own fp32 accumulator (the small planes accumulate
//    apart from the large one) and the logit is hi + (mid + lo) at the end.
// x in LDS: piece-major ([32 pieces][64 tokens + 1] slots of 16 bytes), so
// the 16 lanes of an MFMA row group read 256 contiguous bytes and the
// staging stores of consecutive pieces fall on different banks.  One barrier
// per chunk.  When d_model is a multiple of 256 every chunk is full: its 8
// steps are unrolled without branches (the W_r operands 4 steps ahead come
// from this chunk or, by fixed offsets, the next), so the compiler overlaps
// one step's loads with the previous step's MFMAs; blocks on one
// XCD then also start their walk over the contraction at different chunks.
// Other widths take a general loop.
// MFMA operand layout (16x16x32 bf16): lane l supplies row (l % 16) and the 8
// consecutive k values starting at 8 * (l / 16); result lane l holds column
// (l % 16), rows 4 * (l / 16) + i.
// ---------------------------------------------------------------------------
constexpr int kFwMfmaWaves = 8;
constexpr int kFwStageThreads = 4 * kWave;
constexpr int kFwThreads = kFwMfmaWaves * kWave + kFwStageThreads;  // 768
constexpr int kFwKc = 256;                                          // contraction columns per x chunk
constexpr int kFwPieces = kFwKc / 8;                                // 16-byte pieces of a row per chunk
constexpr int kFwPitch = kRouterTokens + 1;                         // slots per piece (one pad slot)
constexpr int kFwBuf = kFwPieces * kFwPitch * 16;                   // bytes per x buffer
constexpr int kFwStagePer = kRouterTokens * kFwPieces / kFwStageThreads;  // pieces per staging thread
constexpr int kFwRing = 4;                                          // W_r steps in flight per wave

// LDS bytes of the single-pass tail (see route_fused_tail) for N experts
__host__ __device__ constexpr int fused_tail_bytes(int N) { return N * 24 + kRouterTokens * 4 + 16 * 8 + 16; }

// x buffers; after the contraction the logit rows, then (single pass) the
// look-back tail's LDS or (backward) the dx scratch reuse the same bytes
constexpr int kFwSmemX = 2 * kFwBuf > kRouterLgBytes + fused_tail_bytes(kFusedMaxExperts)
                             ? 2 * kFwBuf
                             : (kRouterLgBytes + fused_tail_bytes(kFusedMaxExperts) + 15) / 16 * 16;
struct RouterFwSmem {
  __attribute__((aligned(16))) char x[kFwSmemX];
  uint64_t mask[2][kRouterChunk];  // per route and expert: the block's tokens that chose it (bit t)
  float red[4][kRouterChunk];      // P partial sums of four 16-token groups
  float s_max[kRouterTokens], s_inv[kRouterTokens];
  int s_e[kRouterTokens], s_e2[kRouterTokens];
};
static_assert(kRouterLgBytes <= 2 * kFwBuf, "logit rows fit in the x buffers");

// Workgroup barrier that orders LDS traffic only: each wave waits for its own
// LDS (and scalar memory) operations, then meets the others.  Unlike
// __syncthreads it does not wait for the wave's global loads in flight
// (gfx9 counts loads and stores together, so a release fence would drain the
// W_r register ring and the staging loads at every chunk).  The memory clobber
// keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// The MFMAs of one 32-column step: kTT token tiles x 3 planes.
template <int kTT>
__device__ __forceinline__ void fw_step_mfma(f32x4 (&acc)[3][kTT], const bf16x8 (&a)[kTT], const bf16x8 (&pln)[3]) {
#pragma unroll
  for (int pl = 0; pl < 3; ++pl)
#pragma unroll
    for (int tb = 0; tb < kTT; ++tb)
      acc[pl][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[tb], pln[pl], acc[pl][tb], 0, 0, 0);
}

// kTT: token tiles per MFMA wave.  With all 8 expert tiles of a chunk live
// each wave multiplies its 16 experts for all 4 token tiles; with at most 4
// (N <= 64) or 2 (N <= 32) expert tiles the waves split the block's token
// tiles instead (2 or 4 waves per expert tile, 2 or 1 token tiles each), so
// no wave repeats another's products, and the logit columns past the live
// tiles are set to -inf.
template <bool kLds, int kTT = kTokTiles>
__device__ __forceinline__ LogitRows<kLds> router_fwd_contract_bf16(
    const bf16 *__restrict__ x, const u32x4 *__restrict__ wplanes, const float *__restrict__ bias,
    int64_t T, int d, int N, float *__restrict__ logits_g, int64_t blk, RouterFwSmem &sm) {
  static_assert(kFwStagePer * kFwStageThreads == kRouterTokens * kFwPieces, "staging plan");
  static_assert(kFwMfmaWaves * 16 == kRouterChunk, "16 experts per MFMA wave");
  static_assert(kTT == kTokTiles || (kLds && (kTT == 2 || kTT == 1)), "token tiles per wave");
  constexpr int kTileWaves = kFwMfmaWaves * kTT / kTokTiles;  // waves (= expert tiles) per token group
  const int64_t t0 = blk * kRouterTokens;
  const int nt = (int)min<int64_t>(kRouterTokens, T - t0);
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int nkc = (int)ceil_div(d, kFwKc);            // x chunks per expert chunk
  const int nec = kLds ? 1 : (int)ceil_div(N, kRouterChunk);
  const int Q = nkc * nec;                            // chunks in the walk
  const int S = d / 32;                               // 32-column steps per expert chunk
  const bool full = d % kFwKc == 0;                   // every chunk 8 steps
  const int rot = full ? (int)((blk / 8) % nkc) : 0;

  LogitRows<kLds> lg;
  if (kLds) {
    lg.base = (float *)sm.x;
    lg.stride = kLgStride;
  } else {
    lg.base = logits_g + t0 * N;
    lg.stride = N;
  }

  if (wave >= kFwMfmaWaves) {
    // ---- staging: chunk q of the walk holds columns [kc * 256, ...) of x,
    // kc = (q mod nkc + rot) mod nkc; thread piece u covers row i / 32,
    // piece i mod 32 (i = st + 256 u); pieces past a short chunk's width
    // are loaded clamped and stored to slots no one reads.
    const int st = tid - kFwMfmaWaves * kWave;
    const bf16 *src[kFwStagePer];
    int off[kFwStagePer], pc[kFwStagePer];
#pragma unroll
    for (int u = 0; u < kFwStagePer; ++u) {
      const int i = st + u * kFwStageThreads, r = i / kFwPieces;
      pc[u] = i % kFwPieces;
      src[u] = x + (t0 + min(r, nt - 1)) * d;
      off[u] = (pc[u] * kFwPitch + r) * 16;
    }
    u32x4 ring[2][kFwStagePer];
    auto load = [&](int slot, int q) {
      q = min(q, Q - 1);
      int kc = q % nkc + rot;
      kc = kc >= nkc ? kc - nkc : kc;
      const int c0 = kc * kFwKc, np = min(kFwKc, d - c0) / 8;
#pragma unroll
      for (int u = 0; u < kFwStagePer; ++u) ring[slot][u] = *(const u32x4 *)(src[u] + c0 + min(pc[u], np - 1) * 8);
    };
    auto store = [&](int slot, int buf) {
#pragma unroll
      for (int u = 0; u < kFwStagePer; ++u) *(u32x4 *)(sm.x + buf * kFwBuf + off[u]) = ring[slot][u];
    };
    load(0, 0);
    store(0, 0);
    load(1, 1);
    load(0, 2);
    for (int q = 0; q < Q; ++q) {
      lds_barrier();  // chunk q is in buffer q & 1; buffer (q + 1) & 1 is free
      if (q + 1 < Q) {
        if (q & 1) {
          store(0, 0);
          load(0, q + 3);
        } else {
          store(1, 1);
          load(1, q + 3);
        }
      }
    }
    __syncthreads();  // every MFMA wave is past its last x read
    if (kLds) {       // clear the rank masks for the epilogue
      for (int i = tid - kFwMfmaWaves * kWave; i < 2 * kRouterChunk; i += kFwStageThreads)
        (&sm.mask[0][0])[i] = 0;
      if (kTT < kTokTiles) {  // logit columns past the live expert tiles
        constexpr int kCols = kRouterChunk - kTileWaves * 16;
        for (int i = tid - kFwMfmaWaves * kWave; i < kRouterTokens * kCols; i += kFwStageThreads)
          lg.at(i / kCols, kTileWaves * 16 + i % kCols) = -INFINITY;
      }
    }
  } else {
    // ---- multiply
    const int r16 = lane % 16, kg = lane / 16;
    const int mt = wave % kTileWaves, tb0 = (wave / kTileWaves) * kTT;  // expert tile, first token tile
    f32x4 acc[3][kTT];
    u32x4 pring[kFwRing][3];
    // planes of step g of expert chunk ec: tile ec * 8 + mt (the last tile
    // again past the experts), three contiguous 1 KB pieces, 16 bytes a lane
    const int ntile = (N + 15) / 16;
    auto pl_ptr = [&](int ec, int g) -> const u32x4 * {
      const int m = min(ec * 8 + mt, ntile - 1);
      return wplanes + ((int64_t)m * S + g) * 3 * kWave + lane;
    };
    auto pld = [&](int slot, const u32x4 *p) {
      pring[slot][0] = p[0];
      pring[slot][1] = p[kWave];
      pring[slot][2] = p[2 * kWave];
    };
    auto planes = [&](int slot, bf16x8 (&pln)[3]) {
#pragma unroll
      for (int pl = 0; pl < 3; ++pl) pln[pl] = as_bf16x8(pring[slot][pl]);
    };
    auto write_logits = [&](int ec) {
      // chunk ec's logits (+ bias); in LDS, experts past N get -inf
      const int j = ec * kRouterChunk + mt * 16 + r16;
      const float bj = bias && j < N ? bias[j] : 0.f;
#pragma unroll
      for (int tb = 0; tb < kTT; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = (tb0 + tb) * 16 + kg * 4 + i;
          const float v = acc[0][tb][i] + (acc[1][tb][i] + acc[2][tb][i]) + bj;
          if (kLds)
            lg.at(t, j) = j < N ? v : -INFINITY;
          else if (t < nt && j < N)
            lg.at(t, j) = v;
        }
    };
    auto zero_acc = [&]() {
#pragma unroll
      for (int pl = 0; pl < 3; ++pl)
#pragma unroll
        for (int tb = 0; tb < kTT; ++tb) acc[pl][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    if (full) {
      // chunk q: expert chunk q / nkc, contraction chunk (q mod nkc + rot)
      // mod nkc, whose 8 steps' planes are consecutive
      auto chunk_ptr = [&](int q) -> const u32x4 * {
        q = min(q, Q - 1);
        const int ec = q / nkc;
        int kc = q - ec * nkc + rot;
        kc = kc >= nkc ? kc - nkc : kc;
        return pl_ptr(ec, kc * 8);
      };
      constexpr int kStep = 3 * kWave;  // u32x4 pieces per step
      const u32x4 *cur = chunk_ptr(0);
#pragma unroll
      for (int r = 0; r < kFwRing; ++r) pld(r, cur + r * kStep);
      int kcw = 0, ec = 0;  // position in the expert chunk's walk
      for (int q = 0; q < Q; ++q) {
        const u32x4 *nxt = chunk_ptr(q + 1);  // past the end: this chunk again (never used)
        if (kcw == 0) zero_acc();
        lds_barrier();  // x chunk q is in LDS
        const char *xb = sm.x + (q & 1) * kFwBuf + (kg * kFwPitch + r16) * 16;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          bf16x8 pln[3];
          planes(s % kFwRing, pln);
          pld(s % kFwRing, s + kFwRing < 8 ? cur + (s + kFwRing) * kStep : nxt + (s + kFwRing - 8) * kStep);
          __builtin_amdgcn_sched_barrier(0);  // the refill issues here, 4 steps before its use
          bf16x8 a[kTT];
#pragma unroll
          for (int tb = 0; tb < kTT; ++tb)
            a[tb] = as_bf16x8(*(const u32x4 *)(xb + (s * 4 * kFwPitch + (tb0 + tb) * 16) * 16));
          fw_step_mfma<kTT>(acc, a, pln);
        }
        cur = nxt;
        if (++kcw == nkc) {
          if (!kLds) write_logits(ec);
          kcw = 0;
          ++ec;
        }
      }
    } else {
      // general widths: x chunk g / 8 of the walk, the last one of each
      // expert chunk short
      int gn = 0, ecn = 0;  // next step to fetch (past the last one: the last one again)
      auto fetch_next = [&](int slot) {
        pld(slot, pl_ptr(ecn, gn));
        if (++gn == S) {
          if (ecn + 1 < nec) {
            gn = 0;
            ++ecn;
          } else {
            gn = S - 1;
          }
        }
      };
#pragma unroll
      for (int r = 0; r < kFwRing; ++r) fetch_next(r);
      const int total = nec * S;
      int g = 0, ec = 0, q = 0;  // step within the expert chunk, expert chunk, x chunks started
      for (int G0 = 0; G0 < total; G0 += kFwRing) {
#pragma unroll
        for (int r = 0; r < kFwRing; ++r) {
          if (G0 + r < total) {
            if (g == 0) zero_acc();
            if ((g & 7) == 0) {
              lds_barrier();  // x chunk q is in LDS
              ++q;
            }
            bf16x8 pln[3];
            planes(r, pln);
            fetch_next(r);
            const char *xb = sm.x + ((q - 1) & 1) * kFwBuf + (((g & 7) * 4 + kg) * kFwPitch + r16) * 16;
            bf16x8 a[kTT];
#pragma unroll
            for (int tb = 0; tb < kTT; ++tb) a[tb] = as_bf16x8(*(const u32x4 *)(xb + (tb0 + tb) * 16 * 16));
            fw_step_mfma<kTT>(acc, a, pln);
            if (g == S - 1 && !kLds) write_logits(ec);
            if (++g == S) {
              g = 0;
              ++ec;
            }
          }
        }
      }
    }
    __syncthreads();  // every MFMA wave is past its last x read
    if (kLds) write_logits(0);
  }
  __syncthreads();
  return lg;
}

// W_r split into its three exact bf16 planes (hi + mid + lo, each taking the
// next 8 significant bits) and laid out in MFMA fragment order, once per
// call (or once for good, when the caller keeps W_r in this form): piece (tile m, step g, plane p, lane l) holds the 8 values of expert
// 16 m + l mod 16 (zeros past N) at contraction columns 32 g + 8 (l / 16) ..
// + 8, so each router wave loads its operands of a step as three contiguous
// 1 KB pieces (loads whose consecutive lanes read different rows of W_r
// reach a fraction of the cache bandwidth).  One thread per (m, g, l).
__global__ __launch_bounds__(256) void router_wplanes_kernel(const float *__restrict__ w_r, int N, int d,
                                                             u32x4 *__restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int S = d / 32;
  const int l = (int)(i % kWave);
  const int64_t mg = i / kWave;  // m * S + g
  const int g = (int)(mg % S), m = (int)(mg / S);
  const int row = m * 16 + l % 16;
  f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f}, b = a;
  if (row < N) {
    const float *src = w_r + (int64_t)row * d + g * 32 + (l / 16) * 8;
    a = *(const f32x4 *)src;
    b = *(const f32x4 *)(src + 4);
  }
  bf16x8 hi, mid, lo;
  split3_x8(a, b, hi, mid, lo);
  u32x4 *o = out + mg * 3 * kWave + l;
  o[0] = as_u32x4(hi);
  o[kWave] = as_u32x4(mid);
  o[2 * kWave] = as_u32x4(lo);
}

hipError_t launch_router_planes(const float *w_r, int N, int d, void *wplanes, hipStream_t st) {
  const int64_t n = (int64_t)((N + 15) / 16) * (d / 32) * kWave;
  router_wplanes_kernel<<<dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, st>>>(w_r, N, d, (u32x4 *)wplanes, n);
  return hipGetLastError();
}

// DPP moves within rows of 16 lanes: swap neighbours, swap pairs, mirror the
// 8-lane halves (together a butterfly over each group of 8 lanes).
__device__ __forceinline__ int dpp_xor1(int v) { return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_xor2(int v) { return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_hmirror(int v) { return __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false); }
template <int kStep>
__device__ __forceinline__ int dpp8(int v) {
  return kStep == 0 ? dpp_xor1(v) : kStep == 1 ? dpp_xor2(v) : dpp_hmirror(v);
}
template <int kStep>
__device__ __forceinline__ float dpp8f(float v) {
  return __builtin_bit_cast(float, dpp8<kStep>(__builtin_bit_cast(int, v)));
}

// Epilogue of a router block whose logits (+ bias) sit in LDS rows of
// kLgStride floats, experts past N holding -inf (N <= 128), run by the
// first 512 threads:
//  A. 8 lanes per token, lane q holding experts 32 c + 4 q + i (c, i < 4,
//     four 16-byte reads): the best (and second best) logit and its expert
//     (larger logit first, the lower index on equal logits), the sum of
//     exp(h_j - max) and the probabilities p_j = exp(h_j - max) / sum,
//     written back over the logits; reductions over the 8 lanes by DPP
//     steps (every lane ends with the same bits); each route's choice sets
//     the token's bit in the expert's mask;
//  B. per expert: the block's P partial sum (four 16-token groups, then
//     their sum in a fixed order), its count (bits of the mask) and, per
//     token, the rank among the block's earlier tokens with the same expert
//     (bits of the mask below the token's).
// With s_cnt set (one route per token) the block's counts and P partial sums
// also go to LDS, the sums as 2^-31 fixed point, for the single-pass
// assignment.
template <int kK>
__device__ __forceinline__ void router_epilogue_lds(float *lg, RouterFwSmem &sm, int nt, int N, int64_t t0,
                                                    int64_t blk, TopK tk, int32_t *__restrict__ expert_idx,
                                                    float *__restrict__ gate, int32_t *__restrict__ slot_rank,
                                                    int32_t *__restrict__ bcount, float *__restrict__ ppart,
                                                    int *s_cnt = nullptr, int64_t *s_pfix = nullptr) {
  static_assert(kK == 1 || kK == 2, "one or two routes per token");
  const int tid = threadIdx.x;
  if (tid < kRBThreads) {
    const int t = tid >> 3, q = tid & 7;
    float *row = lg + t * kLgStride + 4 * q;
    float h[16];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4 v = *(const f32x4 *)(row + 32 * c);
#pragma unroll
      for (int i = 0; i < 4; ++i) h[4 * c + i] = v[i];
    }
    float best = -INFINITY, sec = -INFINITY;
    int bi = 0x7fffffff, si = 0x7fffffff;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) topk_take<kK>(h[4 * c + i], 32 * c + 4 * q + i, best, bi, sec, si);
    auto merge = [&](float ov, int oi, float ov2, int oi2) { topk_merge<kK>(ov, oi, ov2, oi2, best, bi, sec, si); };
    merge(dpp8f<0>(best), dpp8<0>(bi), kK == 2 ? dpp8f<0>(sec) : 0.f, kK == 2 ? dpp8<0>(si) : 0);
    merge(dpp8f<1>(best), dpp8<1>(bi), kK == 2 ? dpp8f<1>(sec) : 0.f, kK == 2 ? dpp8<1>(si) : 0);
    merge(dpp8f<2>(best), dpp8<2>(bi), kK == 2 ? dpp8f<2>(sec) : 0.f, kK == 2 ? dpp8<2>(si) : 0);
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      h[k] = expf(h[k] - best);  // exp(-inf) = 0 for the experts past N
      sum += h[k];
    }
    sum += dpp8f<0>(sum);
    sum += dpp8f<1>(sum);
    sum += dpp8f<2>(sum);
    const float inv = 1.0f / sum;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *(f32x4 *)(row + 32 * c) = f32x4{h[4 * c] * inv, h[4 * c + 1] * inv, h[4 * c + 2] * inv, h[4 * c + 3] * inv};
    if (q == 0 && t < nt) {
      sm.s_e[t] = bi;
      expert_idx[t0 + t] = bi;
      gate[t0 + t] = inv;  // p_e = exp(h_e - max) / sum with h_e = max
      __hip_atomic_fetch_or(&sm.mask[0][bi], 1ull << t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (kK == 2) {
        sm.s_e2[t] = si;
        expert_idx[tk.T + t0 + t] = si;
        gate[tk.T + t0 + t] = expf(sec - best) * inv;
        __hip_atomic_fetch_or(&sm.mask[1][si], 1ull << t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
    // B1: P partial sums of 16-token groups (column reads of 64 consecutive experts)
  }
  __syncthreads();
  if (tid < kRBThreads) {
    const int j = tid & (kRouterChunk - 1), r = tid >> 7;
    float p = 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int tt = r * 16 + u;
      if (tt < nt) p += lg[tt * kLgStride + j];
    }
    sm.red[r][j] = p;
  }
  __syncthreads();
  const int64_t Np = count_stride(N);
  if (tid < N) {
    const int j = tid;
    const float p = ((sm.red[0][j] + sm.red[1][j]) + sm.red[2][j]) + sm.red[3][j];
    const int c = __popcll(sm.mask[0][j]);
    ppart[blk * Np + j] = p;
    bcount[blk * Np + j] = c;
    if (kK == 1 && s_cnt) {
      s_cnt[j] = c;
      s_pfix[j] = p_fixed(p);
    }
    if (kK == 2) {
      ppart[(tk.nb + blk) * Np + j] = 0.f;
      bcount[(tk.nb + blk) * Np + j] = __popcll(sm.mask[1][j]);
    }
  }
  if (tid < nt) {
    const uint64_t below = (1ull << tid) - 1;
    slot_rank[t0 + tid] = __popcll(sm.mask[0][sm.s_e[tid]] & below);
    if (kK == 2) slot_rank[tk.nb * kRouterTokens + t0 + tid] = __popcll(sm.mask[1][sm.s_e2[tid]] & below);
  }
}

template <bool kLds, int kK, int kTT = kTokTiles>
__global__ __launch_bounds__(kFwThreads) void router_fwd_bf16_kernel(
    const bf16 *__restrict__ x, const u32x4 *__restrict__ wplanes, const float *__restrict__ bias,
    int64_t T, int d, int N, float *__restrict__ logits_g, int32_t *__restrict__ expert_idx,
    float *__restrict__ gate, int32_t *__restrict__ slot_rank, int32_t *__restrict__ bcount,
    float *__restrict__ ppart) {
  __shared__ RouterFwSmem sm;
  const int64_t blk = blockIdx.x;
  const LogitRows<kLds> lg = router_fwd_contract_bf16<kLds, kTT>(x, wplanes, bias, T, d, N, logits_g, blk, sm);
  const int64_t t0 = blk * kRouterTokens;
  const int nt = (int)min<int64_t>(kRouterTokens, T - t0);
  if (kLds)
    router_epilogue_lds<kK>(lg.base, sm, nt, N, t0, blk, TopK{T, router_blocks(T)}, expert_idx, gate, slot_rank,
                            bcount, ppart);
  else
    router_epilogue<kRBThreads, kLds, kK>(lg, nt, N, t0, blk, TopK{T, router_blocks(T)}, expert_idx, gate,
                                          slot_rank, bcount, ppart, sm.s_max, sm.s_inv, sm.s_e, sm.s_e2);
}

// ---------------------------------------------------------------------------
// fp32 activations: fp32 FMA.  The block's x rows and the chunk's W_r rows are
// staged in LDS in k-slices; each thread owns (token, expert) pairs of the
// current chunk.
// ---------------------------------------------------------------------------
// fp32 logits (+ bias) of block `blk` into `lg` (LDS rows s_lg when
// N <= kRouterChunk, else the global scratch); ends with a barrier.
template <bool kLds>
__device__ __forceinline__ LogitRows<kLds> router_contract_f32(
    const float *__restrict__ x, const float *__restrict__ w_r, const float *__restrict__ bias, int64_t T, int d,
    int N, float *__restrict__ logits_g, int64_t blk, float *s_lg, float (*s_x)[65], float (*s_w)[65]) {
  constexpr int kKc = 64;  // contraction columns per LDS slice
  const int64_t t0 = blk * kRouterTokens;
  const int nt = (int)min<int64_t>(kRouterTokens, T - t0);
  const int tid = threadIdx.x;
  LogitRows<kLds> lg;
  if (kLds) {
    lg.base = s_lg;
    lg.stride = kRouterChunk + 1;
  } else {
    lg.base = logits_g + t0 * N;
    lg.stride = N;
  }
  constexpr int kPer = kRouterTokens * kRouterChunk / kRouterThreads;  // pairs per thread, at most
  for (int c0 = 0; c0 < N; c0 += kRouterChunk) {
    // the chunk's (token, expert) pairs over its live experts only, spread
    // over all threads (with few experts, pairs over the whole chunk width
    // would leave most threads idle and the rest in long serial chains)
    const int nc = min(kRouterChunk, N - c0);
    const int npairs = kRouterTokens * nc;
    float acc[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) acc[q] = 0.f;
    for (int k0 = 0; k0 < d; k0 += kKc) {
      __syncthreads();
      // the slice's x rows and W_r rows (d is a multiple of 64: whole
      // slices), both with coalesced loads issued together
      for (int i = tid; i < kRouterTokens * kKc; i += kRouterThreads) {
        int t = i / kKc, k = i % kKc;
        s_x[t][k] = (t < nt && k0 + k < d) ? x[(t0 + t) * d + k0 + k] : 0.f;
      }
      for (int i = tid; i < nc * kKc; i += kRouterThreads) {
        const int jj = i / kKc, k = i % kKc;
        s_w[jj][k] = w_r[(int64_t)(c0 + jj) * d + k0 + k];
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int pair = tid + q * kRouterThreads;
        if (pair < npairs) {
          const int t = pair / nc, jj = pair % nc;
          float a = acc[q];
#pragma unroll 16
          for (int k = 0; k < kKc; ++k) a = __builtin_fmaf(s_x[t][k], s_w[jj][k], a);
          acc[q] = a;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int pair = tid + q * kRouterThreads;
      if (pair < npairs) {
        const int t = pair / nc, j = c0 + pair % nc;
        if (t < nt) lg.at(t, kLds ? j - c0 : j) = acc[q] + (bias ? bias[j] : 0.f);
      }
    }
    if (kLds) break;
  }
  __syncthreads();
  return lg;
}

template <bool kLds, int kK>
__global__ __launch_bounds__(kRouterThreads) void router_f32_kernel(
    const float *__restrict__ x, const float *__restrict__ w_r, const float *__restrict__ bias,
    int64_t T, int d, int N, float *__restrict__ logits_g, int32_t *__restrict__ expert_idx,
    float *__restrict__ gate, int32_t *__restrict__ slot_rank, int32_t *__restrict__ bcount,
    float *__restrict__ ppart) {
  __shared__ float s_lg[kLds ? kRouterTokens * (kRouterChunk + 1) : 1];
  __shared__ float s_x[kRouterTokens][65];
  __shared__ float s_w[kRouterChunk][65];  // W_r rows of the current slice
  __shared__ float s_max[kRouterTokens], s_inv[kRouterTokens];
  __shared__ int s_e[kRouterTokens], s_e2[kRouterTokens];
  const int64_t blk = blockIdx.x;
  const int64_t t0 = blk * kRouterTokens;
  const int nt = (int)min<int64_t>(kRouterTokens, T - t0);
  const LogitRows<kLds> lg = router_contract_f32<kLds>(x, w_r, bias, T, d, N, logits_g, blk, s_lg, s_x, s_w);
  router_epilogue<kRouterThreads, kLds, kK>(lg, nt, N, t0, blk, TopK{T, router_blocks(T)}, expert_idx, gate,
                                            slot_rank, bcount, ppart, s_max, s_inv, s_e, s_e2);
}

// ---------------------------------------------------------------------------
// Backward ("Switch Routing": the gate keeps the router differentiable; "The
// Load-Balancing Loss": f_i is a hard count without gradient, P_i carries the
// loss's gradient).  One router block per workgroup: the block's logits are
// recomputed exactly as in the forward, then per token
//   dL/dp_j = d_aux N count_j / T^2 + [j = e_t, t kept] dL/dg_t
//   dL/dh_j = p_j (dL/dp_j - sum_i dL/dp_i p_i)
// (dL/dg_t = sum of the expert backward's partial dots <z, H> of token t, in
// a fixed order), written to dh [T][N]; then
//   dx_t = W_r^T dL/dh_t + (W_in^T du)_t (kept t) + dy_t (residual)
// in fp32, one rounding.
// ---------------------------------------------------------------------------
// LDS of the backward epilogue beyond the logit rows: the loss term of dL/dp
// per expert, and per wave a group of kBwdWrCols columns of W_r rows for the
// dx product.
constexpr int kBwdWrCols = 8;
template <int kThreads>
constexpr int bwd_lds_floats() {
  return kRouterChunk + (kThreads / kWave) * kRouterChunk * kBwdWrCols;
}

// kDxHere: form dx in this kernel (fp32 layers, vector ALUs); otherwise
// write the exact bf16 planes of dL/dh for the MFMA dx product (bf16 layers).
template <typename T_, int kThreads, bool kLds, bool kDxHere>
__device__ __forceinline__ void router_bwd_epilogue(const LogitRows<kLds> lg, int nt, int64_t t0, const RouterBwdArgs &a,
                                    float *s_extra) {
  constexpr int kLpt = kThreads / kRouterTokens;  // lanes per token
  constexpr int kW = kThreads / kWave;
  const int N = a.N, d = a.d;
  const int tid = threadIdx.x, t = tid / kLpt, q = tid % kLpt;
  const float caux = a.d_aux * (float)N / ((float)a.T * (float)a.T);
  float *s_aux = s_extra;                // [kRouterChunk] (N <= kRouterChunk)
  float *s_wr = s_extra + kRouterChunk;  // [kW][kRouterChunk][kBwdWrCols]
  if (kLds) {
    if (tid < kThreads)
      for (int j = tid; j < N; j += kThreads) s_aux[j] = caux * (float)a.expert_count[j];
    __syncthreads();
  }
  auto aux = [&](int j) { return kLds ? s_aux[j] : caux * (float)a.expert_count[j]; };
  if (t < nt) {
    const int64_t tt = t0 + t;
    float mx = -INFINITY;
    for (int j = q; j < N; j += kLpt) mx = fmaxf(mx, lg.at(t, j));
#pragma unroll
    for (int off = 1; off < kLpt; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, kWave));
    float sum = 0.f;
    for (int j = q; j < N; j += kLpt) sum += expf(lg.at(t, j) - mx);
#pragma unroll
    for (int off = 1; off < kLpt; off <<= 1) sum += __shfl_xor(sum, off, kWave);
    const float inv = 1.0f / sum;
    const int e = a.expert_idx[tt];
    // dL/dg: the token's partial dots, lane q taking q, q + kLpt, ..., then
    // butterfly steps (the same bits on every lane of the token)
    float dg = 0.f;
    if (!a.dropped[tt])
      for (int i = q; i < a.n_dg; i += kLpt) dg += a.dgpart[tt * a.n_dg + i];
#pragma unroll
    for (int off = 1; off < kLpt; off <<= 1) dg += __shfl_xor(dg, off, kWave);
    float sdp = 0.f;
    for (int j = q; j < N; j += kLpt) {
      const float pj = expf(lg.at(t, j) - mx) * inv;
      const float dp = aux(j) + (j == e ? dg : 0.f);
      lg.at(t, j) = pj;
      sdp += dp * pj;
    }
#pragma unroll
    for (int off = 1; off < kLpt; off <<= 1) sdp += __shfl_xor(sdp, off, kWave);
    for (int j = q; j < N; j += kLpt) {
      const float pj = lg.at(t, j);
      const float dp = aux(j) + (j == e ? dg : 0.f);
      const float dh = pj * (dp - sdp);
      lg.at(t, j) = dh;
      a.dh[tt * N + j] = dh;
      if (!kDxHere) {  // planes in the order hi, hi, mid, hi, lo, mid
        bf16 *ap = (bf16 *)a.aplanes + tt * a.kp + j;
        const bf16 hi = (bf16)dh;
        const float r1 = dh - (float)hi;
        const bf16 mid = (bf16)r1;
        const bf16 lo = (bf16)(r1 - (float)mid);
        ap[0] = hi;
        ap[N] = hi;
        ap[2 * N] = mid;
        ap[3 * N] = hi;
        ap[4 * N] = lo;
        ap[5 * N] = mid;
      }
    }
    if (!kDxHere)  // zero padding of the plane row
      for (int c = 6 * N + q; c < a.kp; c += kLpt) ((bf16 *)a.aplanes)[tt * a.kp + c] = (bf16)0.f;
  }
  __syncthreads();
  // bias partial of the block: sum over its tokens of dL/dh, in token order
  for (int j = tid; j < N && tid < kThreads; j += kThreads) {
    float b = 0.f;
    for (int u = 0; u < nt; ++u) b += lg.at(u, j);
    a.bpart[(t0 / kRouterTokens) * N + j] = b;
  }
  if (!kDxHere) return;
  // dx (fp32 layers): lane = token of the block; wave w takes the column
  // groups w, w + W, ... of kBwdWrCols columns.  With the logits in LDS the
  // wave first copies its group's W_r rows to its own LDS region (each lane
  // then reads them as broadcasts); otherwise the W_r values come straight
  // from memory.
  const int lane = tid % kWave;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int tl = min(lane, nt - 1);
  const int64_t tt = t0 + tl;
  const bool live = lane < nt;
  const bool kept = live && !a.dropped[tt];
  const T_ *dy = (const T_ *)a.dy;
  T_ *dx = (T_ *)a.dx;
  float *wr = s_wr + w * kRouterChunk * kBwdWrCols;
  for (int c0 = w * kBwdWrCols; c0 < d; c0 += kW * kBwdWrCols) {
    if (kLds) {
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the previous group's reads are done
      __builtin_amdgcn_wave_barrier();
      for (int j = lane; j < N; j += kWave) {
        const float *src = a.w_r + (int64_t)j * d + c0;
        *(f32x4 *)(wr + j * kBwdWrCols) = *(const f32x4 *)src;
        *(f32x4 *)(wr + j * kBwdWrCols + 4) = *(const f32x4 *)(src + 4);
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
    }
    float acc[kBwdWrCols];
#pragma unroll
    for (int i = 0; i < kBwdWrCols; ++i) acc[i] = 0.f;
#pragma unroll 4
    for (int j = 0; j < N; ++j) {
      const float h = lg.at(tl, j);
      float wv[kBwdWrCols];
      if (kLds) {
        const f32x4 w0 = *(const f32x4 *)(wr + j * kBwdWrCols), w1 = *(const f32x4 *)(wr + j * kBwdWrCols + 4);
        wv[0] = w0[0]; wv[1] = w0[1]; wv[2] = w0[2]; wv[3] = w0[3];
        wv[4] = w1[0]; wv[5] = w1[1]; wv[6] = w1[2]; wv[7] = w1[3];
      } else {
#pragma unroll
        for (int i = 0; i < kBwdWrCols; ++i) wv[i] = a.w_r[(int64_t)j * d + c0 + i];
      }
#pragma unroll
      for (int i = 0; i < kBwdWrCols; ++i) acc[i] = __builtin_fmaf(h, wv[i], acc[i]);
    }
    if (live) {
#pragma unroll
      for (int i = 0; i < kBwdWrCols; ++i) {
        float v = acc[i];
        if (kept) v += a.dxe[tt * d + c0 + i];
        if (a.add_residual) v += to_f32(dy[tt * d + c0 + i]);
        dx[tt * d + c0 + i] = from_f32<T_>(v);
      }
    }
  }
}

// The logits are recomputed with the forward router's contraction, so they
// are the forward's bits; the epilogue runs on the first 512 threads.
template <bool kLds>
__global__ __launch_bounds__(kFwThreads) void router_bwd_bf16_kernel(const RouterBwdArgs a) {
  __shared__ RouterFwSmem sm;
  const int64_t blk = blockIdx.x, t0 = blk * kRouterTokens;
  const int nt = (int)min<int64_t>(kRouterTokens, a.T - t0);
  const LogitRows<kLds> lg =
      router_fwd_contract_bf16<kLds>((const bf16 *)a.x, (const u32x4 *)a.wplanes, a.bias, a.T, a.d, a.N, a.logits,
                                     blk, sm);
  static_assert(kRouterLgBytes / 4 + bwd_lds_floats<kRBThreads>() <= kFwSmemX / 4,
                "logit rows + backward scratch fit the staging area");
  router_bwd_epilogue<bf16, kRBThreads, kLds, false>(lg, nt, t0, a, (float *)sm.x + kRouterLgBytes / 4);
}

template <bool kLds>
__global__ __launch_bounds__(kRouterThreads) void router_bwd_f32_kernel(const RouterBwdArgs a) {
  __shared__ float s_lg[kLds ? kRouterTokens * (kRouterChunk + 1) : 1];
  __shared__ float s_x[kRouterTokens][65];
  __shared__ float s_w[kRouterChunk][65];  // W_r rows of the current slice
  const int64_t blk = blockIdx.x, t0 = blk * kRouterTokens;
  const int nt = (int)min<int64_t>(kRouterTokens, a.T - t0);
  const LogitRows<kLds> lg =
      router_contract_f32<kLds>((const float *)a.x, a.w_r, a.bias, a.T, a.d, a.N, a.logits, blk, s_lg, s_x, s_w);
  __shared__ __attribute__((aligned(16))) float s_extra[bwd_lds_floats<kRouterThreads>()];
  router_bwd_epilogue<float, kRouterThreads, kLds, true>(lg, nt, t0, a, s_extra);
}

// dW_r = sum_t dh_t x_t^T for fp32 layers: workgroup (j tile, k tile, split
// s) sums tokens [s ts, (s + 1) ts) for a 64 x 64 tile (4 x 4 per thread,
// token chunks of 16 through LDS).  The splits are added in order by
// router_wgrad_sum_kernel.
__global__ __launch_bounds__(256) void router_wgrad_f32_kernel(const float *__restrict__ dh,
                                                               const float *__restrict__ x, int64_t T, int N, int d,
                                                               int64_t ts, float *__restrict__ wpart) {
  __shared__ float sD[16][65], sX[16][65];
  const int j0 = blockIdx.x * 64, k0 = blockIdx.y * 64, sp = blockIdx.z;
  const int64_t ta = min<int64_t>(T, (int64_t)sp * ts), tb = min<int64_t>(T, ta + ts);
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  float acc[4][4] = {};
  for (int64_t c = ta; c < tb; c += 16) {
    for (int i = tid; i < 16 * 64; i += 256) {
      const int r = i / 64, col = i % 64;
      const int64_t t = c + r;
      sD[r][col] = (t < tb && j0 + col < N) ? dh[t * N + j0 + col] : 0.f;
      sX[r][col] = t < tb ? x[t * d + k0 + col] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[i] = sD[k][ty * 4 + i];
        bv[i] = sX[k][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = j0 + ty * 4 + i;
    if (j >= N) continue;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) wpart[((int64_t)sp * N + j) * d + k0 + tx * 4 + jj] = acc[i][jj];
  }
}

// dW_r = sum over the splits of wpart, in order (workgroups [0, wblocks), one
// element per thread, 16 loads in flight); dbias = sum over the router blocks
// of bpart (the following workgroups, one wave per expert: lane l adds blocks
// l, l + 64, ... in order, then the 64 partials meet in a butterfly, which
// every lane evaluates in the same order).  Both are fixed-order sums.
__global__ __launch_bounds__(256) void router_wgrad_sum_kernel(const float *__restrict__ wpart,
                                                               const float *__restrict__ bpart, int N, int d,
                                                               int splits, int64_t nb, int64_t wblocks,
                                                               float *__restrict__ dw_r, float *__restrict__ dbias) {
  if (blockIdx.x < wblocks) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t nd = (int64_t)N * d;
    if (i < nd) {
      float s = 0.f;
#pragma unroll 16
      for (int sp = 0; sp < splits; ++sp) s += wpart[(int64_t)sp * nd + i];
      dw_r[i] = s;
    }
    return;
  }
  const int j = (int)((blockIdx.x - wblocks) * 4 + threadIdx.x / kWave), lane = threadIdx.x % kWave;
  if (j >= N) return;  // whole waves
  float s = 0.f;
#pragma unroll 4
  for (int64_t b = lane; b < nb; b += kWave) s += bpart[b * N + j];
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) s += __shfl_xor(s, off, kWave);
  if (lane == 0) dbias[j] = s;
}

WgradSplit router_wgrad_split(int64_t T, int N, int d) {
  const int64_t tiles = ceil_div(N, 64) * ceil_div(d, 128);
  const int64_t want = std::max<int64_t>(1, std::min<int64_t>(ceil_div(512, tiles), ceil_div(T, 64)));
  WgradSplit w;
  w.ts = std::max<int64_t>(64, ceil_div(ceil_div(T, want), 64) * 64);
  w.splits = (int)std::max<int64_t>(1, ceil_div(T, w.ts));
  return w;
}

hipError_t launch_router_bwd(const RouterBwdArgs &a, hipStream_t st, LaunchMarks marks) {
  auto mark = [&](const char *name) {
    if (marks.fn) marks.fn(marks.ctx, name);
  };
  auto reps = [&]() { return marks.reps ? marks.reps(marks.ctx) : 1; };
  const int64_t nb = router_blocks(a.T);
  const bool lds = a.N <= kRouterChunk;
  for (int r = reps(); r > 0 && nb > 0; --r) {
    if (a.dtype == kBF16) {
      hipError_t e = launch_router_planes(a.w_r, a.N, a.d, a.wplanes, st);
      if (e != hipSuccess) return e;
      (lds ? router_bwd_bf16_kernel<true> : router_bwd_bf16_kernel<false>)<<<dim3((unsigned)nb), dim3(kFwThreads), 0,
                                                                              st>>>(a);
    }
    else
      (lds ? router_bwd_f32_kernel<true> : router_bwd_f32_kernel<false>)<<<dim3((unsigned)nb), dim3(kRouterThreads),
                                                                            0, st>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  mark("bwd_router");
  if (a.dtype == kBF16) {
    RouterDxArgs rd{a.T, a.d, a.N, a.kp, a.w_r, a.aplanes, a.bplanes, a.dxe, a.dropped,
                    a.add_residual ? a.dy : nullptr, a.dx};
    for (int r = reps(); r > 0 && e == hipSuccess; --r) e = launch_router_dx_bf16(rd, st);
    if (e != hipSuccess) return e;
  }
  mark("bwd_router_dx");
  const WgradSplit sp = router_wgrad_split(a.T, a.N, a.d);
  for (int r = reps(); r > 0 && e == hipSuccess; --r) {
    if (a.dtype == kBF16) {
      e = launch_router_wgrad_bf16(a.dh, a.x, a.T, a.N, a.d, sp, a.wpart, st);
    } else {
      const dim3 g((unsigned)ceil_div(a.N, 64), (unsigned)(a.d / 64), (unsigned)sp.splits);
      router_wgrad_f32_kernel<<<g, dim3(256), 0, st>>>(a.dh, (const float *)a.x, a.T, a.N, a.d, sp.ts, a.wpart);
      e = hipGetLastError();
    }
  }
  if (e != hipSuccess) return e;
  mark("bwd_router_w");
  const int64_t nd = (int64_t)a.N * a.d;
  const int64_t wblocks = ceil_div(nd, 256), bblocks = a.dbias ? ceil_div(a.N, 4) : 0;
  for (int r = reps(); r > 0; --r)
    router_wgrad_sum_kernel<<<dim3((unsigned)(wblocks + bblocks)), dim3(256), 0, st>>>(
        a.wpart, a.bpart, a.N, a.d, sp.splits, nb, wblocks, a.dw_r, a.dbias);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  mark("bwd_router_w_sum");
  return hipSuccess;
}

template <int kK>
hipError_t run_router(const RouteArgs &a, hipStream_t st) {
  const int64_t nb = router_blocks(a.T);
  const bool lds = a.N <= kRouterChunk;
  const dim3 grid((unsigned)nb);
  if (a.dtype == kBF16) {
    if (!a.wr_planes) {
      hipError_t e = launch_router_planes(a.w_r, a.N, a.d, a.wplanes, st);
      if (e != hipSuccess) return e;
    }
    // at most 2 or 4 live expert tiles: the waves split the token tiles
    const int ntile = (a.N + 15) / 16;
    auto kern = !lds       ? router_fwd_bf16_kernel<false, kK>
                : ntile <= 2 ? router_fwd_bf16_kernel<true, kK, 1>
                : ntile <= 4 ? router_fwd_bf16_kernel<true, kK, 2>
                             : router_fwd_bf16_kernel<true, kK>;
    kern<<<grid, dim3(kFwThreads), 0, st>>>((const bf16 *)a.x, (const u32x4 *)a.wplanes, a.bias, a.T, a.d, a.N,
                                            a.logits, a.expert_idx, a.gate, a.rank, a.bcount, a.ppart);
  } else {
    auto kern = lds ? router_f32_kernel<true, kK> : router_f32_kernel<false, kK>;
    kern<<<grid, dim3(kRouterThreads), 0, st>>>((const float *)a.x, a.w_r, a.bias, a.T, a.d, a.N, a.logits,
                                                a.expert_idx, a.gate, a.rank, a.bcount, a.ppart);
  }
  return hipGetLastError();
}

hipError_t launch_router(const RouteArgs &a, hipStream_t st) {
  if (router_blocks(a.T) == 0) return hipSuccess;
  return a.k == 2 ? run_router<2>(a, st) : run_router<1>(a, st);
}

// ---------------------------------------------------------------------------
// Single-pass routing ("Expert Capacity and the Capacity Factor": slots in
// token order; "The Load-Balancing Loss"), one route per token: each block
// routes its 64 tokens as above, then assigns their slots itself, so x is
// read once and, with a dispatch buffer, each kept row is copied to
// dispatched[e][slot] from the copy of it the block loaded before it waited.
//
// Token order across blocks comes from a decoupled look-back.  Block b
// (state[b]: 0 nothing yet, 1 aggregate, 2 inclusive prefix):
//   1. writes its counts and P sums (aggregate) and sets state 1;
//   2. wave 0 reads the states of the 64 nearest earlier blocks at once and,
//      once every block up to the nearest inclusive one (or the whole window)
//      has published, all threads add those rows; repeated until an
//      inclusive prefix or block 0 is reached;
//   3. writes exclusive + aggregate as its inclusive prefix, state 2;
//   4. slot = exclusive count of the expert + in-block rank, dropped, and the
//      dispatch stores;
//   5. the last block forms the totals and the loss from its inclusive row.
// Ordering across the XCDs follows the HIP memory model at agent scope: a
// block's row stores happen before (a workgroup barrier, then) thread 0's
// release store of the state word that announces them; the look-back reads
// state words with relaxed agent-scope loads and, once it has seen every
// state it needs, runs an agent-scope acquire fence before any thread reads
// those rows (a relaxed load that reads a released value, then an acquire
// fence, synchronises with the release).  Counts are integers and P sums 2^-31 fixed-point
// integers, so every total is independent of how the look-back grouped the
// blocks.  A workgroup takes its router block from an atomic ticket, so every
// block it waits for belongs to a workgroup that is already running and never
// waits for a later one: the chain always drains.  Each wait is bounded: one
// that gives up (not reached by a correct launch) sets the error word and the
// loss to NaN and goes on, so the kernel always ends.  A small kernel clears
// the ticket, the error word and the states before every launch.
// ---------------------------------------------------------------------------
constexpr int kSpinLimit = 1 << 20;  // polls (~1 s)

__global__ __launch_bounds__(256) void route_sync_clear_kernel(u32x4 *__restrict__ p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    p[i] = u32x4{0, 0, 0, 0};
}

// LDS of the single-pass tail (after the logit rows, which the epilogue
// reads until its end).
struct TailLds {
  int64_t *p, *xp;  // [N] block P sums, exclusive P sums (fixed point)
  int *c, *xc;      // [N] block counts, exclusive counts
  int *dst;         // [kRouterTokens] destination row e * C + slot, or -1
  double *red;      // [16] loss partials of the waves
  int *win;         // [2] look-back window: rows to add, last one inclusive
};
__device__ __forceinline__ TailLds tail_lds(char *base, int N) {
  TailLds L;
  L.p = (int64_t *)base;
  L.xp = L.p + N;
  L.red = (double *)(L.xp + N);
  L.c = (int *)(L.red + 16);
  L.xc = L.c + N;
  L.dst = L.xc + N;
  L.win = L.dst + kRouterTokens;
  return L;
}

// Wave 0: states of blocks lo - 1 - lane.  Returns how many of them to add
// (through the nearest one with an inclusive prefix, else all of the window)
// once each of those has published; `found` says the last of them is
// inclusive.  Every decision is a ballot, so the loop is wave-uniform.
__device__ __forceinline__ int lookback_window(const int32_t *state, int64_t lo, int32_t *err, bool &found) {
  const int lane = threadIdx.x % kWave;
  const int64_t j = lo - 1 - lane;
  const int nvalid = (int)min<int64_t>(lo, kWave);
  for (int it = 0;; ++it) {
    const int st = __hip_atomic_load(state + (j > 0 ? j : 0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long inc = __ballot(lane < nvalid && st == 2);
    const int n = inc ? __ffsll(inc) : nvalid;
    const unsigned long long miss = __ballot(lane < n && st == 0);
    if (!miss) {
      found = inc != 0;
      return n;
    }
    // give up after kSpinLimit polls, or at once when another wait already did
    const bool quit = it == kSpinLimit ||
                      ((it & 255) == 255 &&
                       __builtin_amdgcn_readfirstlane(__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)));
    if (quit) {
      if (lane == 0) __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      found = false;
      return n;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Steps 1-5 for block blk (its tokens' experts in s_e, in-block ranks in
// r.slot, counts and P sums in L.c / L.p).
template <int kThreads>
__device__ __forceinline__ void route_fused_tail(const FusedRouteArgs &a, int64_t blk, int64_t nb, int nt, const int *s_e,
                                 const TailLds L) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int N = a.r.N;
  const int64_t Ns = a.row_stride, t0 = blk * kRouterTokens;
  int32_t *const state = a.sync + 4;

  __syncthreads();  // the epilogue's LDS rows are complete
  // 1. aggregate (block 0: its inclusive prefix)
  {
    int32_t *rc = (blk == 0 ? a.inc_c : a.agg_c) + blk * Ns;
    int64_t *rp = (blk == 0 ? a.inc_p : a.agg_p) + blk * Ns;
    for (int e = tid; e < N; e += kThreads) {
      rc[e] = L.c[e];
      rp[e] = L.p[e];
      L.xc[e] = 0;
      L.xp[e] = 0;
    }
  }
  __syncthreads();  // every thread's row stores happen before thread 0's release
  if (tid == 0) __hip_atomic_store(state + blk, blk == 0 ? 2 : 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);

  // the dispatch copy's first kU pieces per thread, loaded now so that they
  // arrive while the block waits for the blocks before it
  constexpr int kU = 12;
  const int row16 = a.r.d * (a.r.dtype == kBF16 ? 2 : 4) / 16;
  const u32x4 *xs = (const u32x4 *)a.r.x + t0 * row16;
  u32x4 *ds = (u32x4 *)a.dispatched;
  const int items = nt * row16;
  u32x4 v[kU];
  if (ds) {
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = xs[min(u * kThreads + tid, items - 1)];
  }

  // 2. look-back: G threads per expert share a window's rows
  const int G = N >= kThreads ? 1 : kThreads / N;
  const int q = tid / min(N, kThreads);
  int64_t lo = blk;
  while (lo > 0) {
    if (wave == 0) {
      bool found;
      const int n = lookback_window(state, lo, a.sync + 1, found);
      // the states just read were stored with release semantics: this fence
      // makes every row those blocks wrote before them visible to the reads
      // below (the barrier orders the other waves' reads after it)
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      if (lane == 0) {
        L.win[0] = n;
        L.win[1] = found ? 1 : 0;
      }
    }
    __syncthreads();
    const int n = L.win[0];
    const bool found = L.win[1] != 0;
    if (q < G) {
      for (int e = tid % min(N, kThreads); e < N; e += kThreads) {
        int c = 0;
        int64_t p = 0;
#pragma unroll 4
        for (int l = q; l < n; l += G) {
          const int64_t j = lo - 1 - l;
          const bool inc = found && l == n - 1;
          c += (inc ? a.inc_c : a.agg_c)[j * Ns + e];
          p += (inc ? a.inc_p : a.agg_p)[j * Ns + e];
        }
        if (c) atomicAdd(&L.xc[e], c);
        if (p) atomicAdd((unsigned long long *)&L.xp[e], (unsigned long long)p);
      }
    }
    __syncthreads();
    lo = found ? 0 : lo - n;
  }

  // 3. inclusive prefix of this block
  if (blk > 0) {
    for (int e = tid; e < N; e += kThreads) {
      a.inc_c[blk * Ns + e] = L.xc[e] + L.c[e];
      a.inc_p[blk * Ns + e] = L.xp[e] + L.p[e];
    }
    __syncthreads();
    if (tid == 0) __hip_atomic_store(state + blk, 2, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }

  // slots and drops
  const int C = a.r.C;
  if (tid < nt) {
    const int e = s_e[tid];
    const int sl = L.xc[e] + a.r.slot[t0 + tid];  // the epilogue left the in-block rank there
    const bool drop = sl >= C;
    a.r.slot[t0 + tid] = sl;
    a.r.dropped[t0 + tid] = drop ? 1 : 0;
    L.dst[tid] = drop ? -1 : e * C + sl;
  }
  __syncthreads();

  // dispatch: the loaded pieces, then the rest of the block's rows
  if (ds) {
    for (int b = 0; b < items; b += kThreads * kU) {
      if (b > 0) {
#pragma unroll
        for (int u = 0; u < kU; ++u) v[u] = xs[min(b + u * kThreads + tid, items - 1)];
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i = b + u * kThreads + tid;
        if (i < items) {
          const int t = i / row16;
          const int dst = L.dst[t];
          if (dst >= 0) ds[(int64_t)dst * row16 + (i - t * row16)] = v[u];
        }
      }
    }
  }

  // totals and loss: N sum_i (count_i / T) (P_i / T), in double, fixed order
  if (blk == nb - 1) {
    double acc = 0.0;
    for (int e = tid; e < N; e += kThreads) {
      const int tot = L.xc[e] + L.c[e];
      a.r.expert_count[e] = tot;
      acc += (double)tot * (double)(L.xp[e] + L.p[e]);
    }
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) acc += __shfl_xor(acc, off, kWave);
    if (lane == 0) L.red[wave] = acc;
    __syncthreads();
    if (tid == 0) {
      double sum = 0.0;
      for (int w = 0; w < kThreads / kWave; ++w) sum += L.red[w];
      const double tt = (double)a.r.T;
      const bool bad = __hip_atomic_load(a.sync + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
      a.r.aux_loss[0] = bad ? __builtin_nanf("") : (float)(sum * 0x1p-31 * (double)N / (tt * tt));
    }
  }
}

// The block's ticket; past the grid (a launch whose ticket was not cleared)
// the workgroup does nothing.
__device__ __forceinline__ int64_t route_ticket(int32_t *ticket, int *s_blk) {
  if (threadIdx.x == 0) *s_blk = __hip_atomic_fetch_add(ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  return *s_blk;
}

template <bool kLds>
__global__ __launch_bounds__(kFwThreads) void route_fused_bf16_kernel(const FusedRouteArgs a) {
  static_assert(kRouterLgBytes + fused_tail_bytes(kFusedMaxExperts) <= kFwSmemX, "tail LDS");
  __shared__ RouterFwSmem sm;
  __shared__ int s_blk;
  const int64_t T = a.r.T, nb = router_blocks(T);
  const int64_t blk = route_ticket(a.sync, &s_blk);
  if (blk >= nb) return;
  const int N = a.r.N;
  const LogitRows<kLds> lg =
      router_fwd_contract_bf16<kLds>((const bf16 *)a.r.x, (const u32x4 *)a.r.wplanes, a.r.bias, T, a.r.d, N,
                                     a.r.logits, blk, sm);
  const int64_t t0 = blk * kRouterTokens;
  const int nt = (int)min<int64_t>(kRouterTokens, T - t0);
  const TailLds L = tail_lds(sm.x + kRouterLgBytes, N);
  if (kLds)
    router_epilogue_lds<1>(lg.base, sm, nt, N, t0, blk, TopK{T, nb}, a.r.expert_idx, a.r.gate, a.r.slot,
                           a.r.bcount, a.r.ppart, L.c, L.p);
  else
    router_epilogue<kRBThreads, kLds, 1>(lg, nt, N, t0, blk, TopK{T, nb}, a.r.expert_idx, a.r.gate, a.r.slot,
                                         a.r.bcount, a.r.ppart, sm.s_max, sm.s_inv, sm.s_e, sm.s_e2, L.c, L.p);
  route_fused_tail<kFwThreads>(a, blk, nb, nt, sm.s_e, L);
}

template <bool kLds>
__global__ __launch_bounds__(kRouterThreads) void route_fused_f32_kernel(const FusedRouteArgs a) {
  constexpr int kLg = kLds ? kRouterTokens * (kRouterChunk + 1) * 4 : 0;
  constexpr int kX = kRouterTokens * 65 * 4;
  constexpr int kTail = fused_tail_bytes(kFusedMaxExperts);
  __shared__ __attribute__((aligned(16))) char s_buf[kLg + (kX > kTail ? kX : kTail)];
  __shared__ float s_w[kRouterChunk][65];  // W_r rows of the current slice
  __shared__ float s_max[kRouterTokens], s_inv[kRouterTokens];
  __shared__ int s_e[kRouterTokens], s_e2[kRouterTokens];
  __shared__ int s_blk;
  const int64_t T = a.r.T, nb = router_blocks(T);
  const int64_t blk = route_ticket(a.sync, &s_blk);
  if (blk >= nb) return;
  const int N = a.r.N;
  const int64_t t0 = blk * kRouterTokens;
  const int nt = (int)min<int64_t>(kRouterTokens, T - t0);
  const LogitRows<kLds> lg = router_contract_f32<kLds>((const float *)a.r.x, a.r.w_r, a.r.bias, T, a.r.d, N,
                                                       a.r.logits, blk, (float *)s_buf,
                                                       (float(*)[65])(s_buf + kLg), s_w);
  const TailLds L = tail_lds(s_buf + kLg, N);  // the x slices are dead after the contraction
  router_epilogue<kRouterThreads, kLds, 1>(lg, nt, N, t0, blk, TopK{T, nb}, a.r.expert_idx, a.r.gate, a.r.slot,
                                           a.r.bcount, a.r.ppart, s_max, s_inv, s_e, s_e2, L.c, L.p);
  route_fused_tail<kRouterThreads>(a, blk, nb, nt, s_e, L);
}

hipError_t launch_route_fused(const FusedRouteArgs &a, hipStream_t st, LaunchMarks marks) {
  const int64_t nb = router_blocks(a.r.T);
  if (nb == 0) return launch_assign(a.r, LayerMaps{}, st, marks);  // no tokens: zero totals and loss
  const bool lds = a.r.N <= kRouterChunk;
  const int64_t n16 = (int64_t)(a.clear_bytes / 16);
  const int reps = marks.reps ? marks.reps(marks.ctx) : 1;
  for (int r = reps; r > 0; --r) {
    route_sync_clear_kernel<<<dim3((unsigned)std::min<int64_t>(ceil_div(n16, 256), 2048)), dim3(256), 0, st>>>(
        (u32x4 *)a.sync, n16);
    if (a.r.dtype == kBF16) {
      if (!a.r.wr_planes) {
        hipError_t e = launch_router_planes(a.r.w_r, a.r.N, a.r.d, a.r.wplanes, st);
        if (e != hipSuccess) return e;
      }
      auto kern = lds ? route_fused_bf16_kernel<true> : route_fused_bf16_kernel<false>;
      kern<<<dim3((unsigned)nb), dim3(kFwThreads), 0, st>>>(a);
    } else {
      auto kern = lds ? route_fused_f32_kernel<true> : route_fused_f32_kernel<false>;
      kern<<<dim3((unsigned)nb), dim3(kRouterThreads), 0, st>>>(a);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (marks.fn) marks.fn(marks.ctx, "route_fused");
  return hipSuccess;
}

}  // namespace smx
