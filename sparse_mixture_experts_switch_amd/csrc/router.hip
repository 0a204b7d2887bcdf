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
// significant bits; every block splits the fp32 rows as it stages them), so
// every product x_k * plane_k is exact in fp32 and the fp32 accumulation sees
// the same terms as an fp32 dot product.
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

template <int kK>
__device__ __forceinline__ void topk_take(float h, int j, float &b1, int &i1, float &b2, int &i2) {
  // ascending j within one lane: strict comparisons keep the lower index
  if (h > b1) {
    if (kK == 2) {
      b2 = b1;
      i2 = i1;
    }
    b1 = h;
    i1 = j;
  } else if (kK == 2 && h > b2) {
    b2 = h;
    i2 = j;
  }
}

__device__ __forceinline__ bool topk_before(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// With s_cnt set (one route per token) the block's counts and P partial sums
// also go to LDS, the sums as 2^-31 fixed point (s_pfix), for the single-pass
// assignment that follows in the same kernel.
template <int kThreads, bool kLds, int kK>
__device__ void router_epilogue(const LogitRows<kLds> lg, int nt, int N, int64_t t0, int64_t blk, TopK tk,
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
      if (kK == 2) {
        // top two of the union of two ordered pairs
        const float ov2 = __shfl_xor(sec, off, kWave);
        const int oi2 = __shfl_xor(si, off, kWave);
        if (topk_before(ov, oi, best, bi)) {  // theirs first; second: my first or their second
          const bool mine = topk_before(best, bi, ov2, oi2);
          sec = mine ? best : ov2;
          si = mine ? bi : oi2;
          best = ov;
          bi = oi;
        } else if (topk_before(ov, oi, sec, si)) {  // mine first; second: their first or my second
          sec = ov;
          si = oi;
        }
      } else if (topk_before(ov, oi, best, bi)) {
        best = ov;
        bi = oi;
      }
    }
    float sum = 0.f;
    if (kLds) {
      constexpr int kJ = kRouterChunk / kLpt;
      float ev[kJ];
#pragma unroll
      for (int i = 0; i < kJ; ++i) ev[i] = q + i * kLpt < N ? __expf(lg.at(t, q + i * kLpt) - best) : 0.f;
#pragma unroll
      for (int i = 0; i < kJ; ++i) {
        if (q + i * kLpt < N) lg.at(t, q + i * kLpt) = ev[i];
        sum += ev[i];
      }
    } else {
      for (int j = q; j < N; j += kLpt) {
        const float ev = __expf(lg.at(t, j) - best);
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
        gate[tk.T + t0 + t] = __expf(sec - best) * inv;
      }
    }
  }
  __syncthreads();
  const int64_t Np = count_stride(N);
  for (int j0 = 0; j0 < N; j0 += kRouterChunk) {
    const int j = j0 + tid / kTpe, r = tid % kTpe;
    float p = 0.f;
    int c = 0, c2 = 0;
    if (j < N) {
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
    if (r == 0 && j < N) {
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

// ---------------------------------------------------------------------------
// bf16 activations, 3-plane bf16 MFMA (v_mfma_f32_16x16x32_bf16).
// 8 waves in two roles, one of each on every SIMD, so that staging and
// matrix work overlap instead of taking turns:
//  - waves 4..7 stage: they load the block's 64 token rows (bf16) and the
//    fp32 rows of a 128-expert chunk of W_r 64 contraction columns at a time
//    (row-contiguous loads, a register ring up to two chunks ahead) and write
//    them to a padded LDS buffer;
//  - waves 0..3 multiply: wave w computes experts [c0 + 32w, c0 + 32w + 32)
//    for all 64 tokens (4 token tiles x 2 expert tiles of 16x16) from the
//    other LDS buffer, splitting its W_r operands into the three bf16 planes
//    as it reads them (fp32 in LDS costs fewer bytes than three planes).
// One barrier per chunk swaps the two buffers.  Every block reads the same
// W_r rows (from L2); the blocks of one XCD start their walk over the
// contraction at different chunks so that they do not all ask for the same
// cache lines at once.
// MFMA operand layout (16x16x32): lane l supplies row (l % 16) and the 8
// consecutive k values starting at 8 * (l / 16); the result lane l holds
// column (l % 16), rows 4 * (l / 16) + i.
// ---------------------------------------------------------------------------
constexpr int kRBThreads = 512;
constexpr int kStageThreads = 256;           // waves 4..7
constexpr int kTokTiles = kRouterTokens / 16;
constexpr int kRKC = 64;                     // contraction columns per chunk
constexpr int kRLS = kRKC + 8;               // padded LDS row of x (bf16)
constexpr int kWLS = kRKC + 4;               // padded LDS row of W_r (fp32)
constexpr int kXPer = kRouterTokens * (kRKC / 8) / kStageThreads;  // 16-byte x pieces per staging thread
constexpr int kWGrp = kRouterChunk * (kRKC / 8) / kStageThreads;   // 8-value W_r groups per staging thread
constexpr int kXStage = kRouterTokens * kRLS * 2;                  // bytes per x stage
constexpr int kWStage = kRouterChunk * kWLS * 4;                   // bytes per W_r stage
constexpr int kRouterStageBytes = 2 * (kXStage + kWStage);
constexpr int kRouterLgBytes = kRouterTokens * (kRouterChunk + 1) * 4;
constexpr int kRouterSmem = kRouterStageBytes > kRouterLgBytes ? kRouterStageBytes : kRouterLgBytes;

// LDS of one router block (bf16 path).
struct RouterSmem {
  __attribute__((aligned(16))) char stage[kRouterSmem];
  float s_max[kRouterTokens], s_inv[kRouterTokens];
  int s_e[kRouterTokens], s_e2[kRouterTokens];
};

// Logits (+ bias) of block `blk` (tokens [64 blk, 64 blk + 64)) into LDS
// (N <= kRouterChunk) or the block's rows of the global scratch; returns
// after a barrier with the logits complete.  Starts with a barrier, so
// consecutive calls by one workgroup may reuse `sm`.
template <bool kLds>
__device__ __forceinline__ LogitRows<kLds> router_contract_bf16(
    const bf16 *__restrict__ x, const float *__restrict__ w_r, const float *__restrict__ bias,
    int64_t T, int d, int N, float *__restrict__ logits_g, int64_t blk, RouterSmem &sm) {
  static_assert(kRBThreads == 8 * kWave && kStageThreads == 4 * kWave && kRouterChunk == 128,
                "4 MFMA waves x 32 experts + 4 staging waves");
  static_assert(kXPer * kStageThreads == kRouterTokens * (kRKC / 8), "x pieces");
  static_assert(kWGrp * kStageThreads == kRouterChunk * (kRKC / 8), "W_r groups");
  char *const smem = sm.stage;
  char *xs = smem;                    // [2][64][kRLS] bf16
  char *ws = smem + 2 * kXStage;      // [2][128][kWLS] fp32

  constexpr int kRing = kLds ? 3 : 2;  // register ring depth of the staging waves
  const int64_t t0 = blk * kRouterTokens;
  const int nt = (int)min<int64_t>(kRouterTokens, T - t0);
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const bool stager = wave >= 4;  // wave-uniform role
  const int ptid = tid - kStageThreads;
  const int r16 = lane % 16, kq = (lane / 16) * 8;
  const int nk = d / kRKC;
  const int rot = (int)((blk / 8) % nk);  // first chunk of this block's walk (blocks b, b + 8, ... share an XCD)

  LogitRows<kLds> lg;
  if (kLds) {
    lg.base = (float *)smem;  // reuses the staging buffers after the contraction
    lg.stride = kRouterChunk + 1;
  } else {
    lg.base = logits_g + t0 * N;
    lg.stride = N;
  }

  // Staging plan.  x: piece i covers 16 bytes of token row i / 8.  W_r:
  // group g covers 8 consecutive fp32 values of expert row g / 8.
  const bf16 *xsrc[kXPer];
  int xoff[kXPer];
#pragma unroll
  for (int q = 0; q < kXPer; ++q) {
    const int i = max(ptid, 0) + q * kStageThreads, r = i / 8, c = i % 8;
    xsrc[q] = x + (t0 + min(r, nt - 1)) * d + c * 8;
    xoff[q] = (r * kRLS + c * 8) * 2;
  }

  for (int c0 = 0; c0 < N; c0 += kRouterChunk) {
    const float *wsrc[kWGrp];
    int woff[kWGrp];
#pragma unroll
    for (int q = 0; q < kWGrp; ++q) {
      const int g = max(ptid, 0) + q * kStageThreads, e = g / 8, c = g % 8;
      wsrc[q] = w_r + (int64_t)min(c0 + e, N - 1) * d + c * 8;
      woff[q] = (e * kWLS + c * 8) * 4;
    }
    u32x4 xr[kRing][kXPer];
    f32x4 wr[kRing][kWGrp][2];
    // chunk ch of the walk (ch >= nk: a repeat of the last one, never used)
    auto fetch = [&](int slot, int ch) {
      int kc = min(ch, nk - 1) + rot;
      kc = (kc >= nk ? kc - nk : kc) * kRKC;
#pragma unroll
      for (int q = 0; q < kXPer; ++q) xr[slot][q] = *(const u32x4 *)(xsrc[q] + kc);
#pragma unroll
      for (int q = 0; q < kWGrp; ++q) {
        wr[slot][q][0] = *(const f32x4 *)(wsrc[q] + kc);
        wr[slot][q][1] = *(const f32x4 *)(wsrc[q] + kc + 4);
      }
    };
    auto store = [&](int slot, int buf) {
#pragma unroll
      for (int q = 0; q < kXPer; ++q) *(u32x4 *)(xs + buf * kXStage + xoff[q]) = xr[slot][q];
#pragma unroll
      for (int q = 0; q < kWGrp; ++q) {
        *(f32x4 *)(ws + buf * kWStage + woff[q]) = wr[slot][q][0];
        *(f32x4 *)(ws + buf * kWStage + woff[q] + 16) = wr[slot][q][1];
      }
    };
    f32x4 acc[kTokTiles][2];
#pragma unroll
    for (int tb = 0; tb < kTokTiles; ++tb) acc[tb][0] = acc[tb][1] = f32x4{0.f, 0.f, 0.f, 0.f};

    __syncthreads();  // previous chunk's readers of the staging buffers are done
    if (stager) {
#pragma unroll
      for (int j = 0; j < kRing; ++j) fetch(j, j);
      store(0, 0);
    }
    __syncthreads();
    for (int base = 0; base < nk; base += kRing) {
#pragma clang loop unroll(full)
      for (int j = 0; j < kRing; ++j) {
        const int ch = base + j;
        if (stager) {
          // slot j held chunk ch, already in LDS: refill it kRing chunks
          // ahead, then move chunk ch + 1 into the other LDS buffer
          fetch(j, ch + kRing);
          store((j + 1) % kRing, (ch + 1) & 1);
        } else if (ch < nk) {
          const bf16 *xb = (const bf16 *)(xs + (ch & 1) * kXStage);
          const float *wbuf = (const float *)(ws + (ch & 1) * kWStage);
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            bf16x8 b[2][3], a[kTokTiles];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const float *src = wbuf + (wave * 32 + q * 16 + r16) * kWLS + s * 32 + kq;
              split3_x8(*(const f32x4 *)src, *(const f32x4 *)(src + 4), b[q][0], b[q][1], b[q][2]);
            }
#pragma unroll
            for (int tb = 0; tb < kTokTiles; ++tb)
              a[tb] = as_bf16x8(*(const u32x4 *)(xb + (tb * 16 + r16) * kRLS + s * 32 + kq));
#pragma unroll
            for (int pl = 0; pl < 3; ++pl)
#pragma unroll
              for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int tb = 0; tb < kTokTiles; ++tb)
                  acc[tb][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[tb], b[q][pl], acc[tb][q], 0, 0, 0);
          }
        }
        __syncthreads();
      }
    }
    // scatter each MFMA wave's 64 x 32 logits tile (the staging buffers are
    // free: the loop ended with a barrier)
    if (!stager) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int j = c0 + wave * 32 + q * 16 + r16;
        if (j < N) {
          const float bj = bias ? bias[j] : 0.f;
#pragma unroll
          for (int tb = 0; tb < kTokTiles; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int t = tb * 16 + (lane / 16) * 4 + i;
              if (t < nt) lg.at(t, kLds ? j - c0 : j) = acc[tb][q][i] + bj;
            }
        }
      }
    }
    if (kLds) break;  // N <= kRouterChunk: one chunk holds every expert
  }
  __syncthreads();
  return lg;
}

// Router work of block `blk`: logits, then the forward epilogue.
template <bool kLds, int kK>
__device__ __forceinline__ void router_block_bf16(
    const bf16 *__restrict__ x, const float *__restrict__ w_r, const float *__restrict__ bias,
    int64_t T, int d, int N, float *__restrict__ logits_g, int32_t *__restrict__ expert_idx,
    float *__restrict__ gate, int32_t *__restrict__ slot_rank, int32_t *__restrict__ bcount,
    float *__restrict__ ppart, int64_t blk, RouterSmem &sm) {
  const LogitRows<kLds> lg = router_contract_bf16<kLds>(x, w_r, bias, T, d, N, logits_g, blk, sm);
  const int64_t t0 = blk * kRouterTokens;
  const int nt = (int)min<int64_t>(kRouterTokens, T - t0);
  router_epilogue<kRBThreads, kLds, kK>(lg, nt, N, t0, blk, TopK{T, router_blocks(T)}, expert_idx, gate, slot_rank,
                                        bcount, ppart, sm.s_max, sm.s_inv, sm.s_e, sm.s_e2);
}

template <bool kLds, int kK>
__global__ __launch_bounds__(kRBThreads) void router_bf16_kernel(
    const bf16 *__restrict__ x, const float *__restrict__ w_r, const float *__restrict__ bias,
    int64_t T, int d, int N, float *__restrict__ logits_g, int32_t *__restrict__ expert_idx,
    float *__restrict__ gate, int32_t *__restrict__ slot_rank, int32_t *__restrict__ bcount,
    float *__restrict__ ppart) {
  __shared__ RouterSmem sm;
  router_block_bf16<kLds, kK>(x, w_r, bias, T, d, N, logits_g, expert_idx, gate, slot_rank, bcount, ppart,
                              blockIdx.x, sm);
}

// ---------------------------------------------------------------------------
// fp32 activations: fp32 FMA.  The block's x rows are staged in LDS in
// k-slices; each thread owns (token, expert) pairs of the current chunk.
// ---------------------------------------------------------------------------
// fp32 logits (+ bias) of block `blk` into `lg` (LDS rows s_lg when
// N <= kRouterChunk, else the global scratch); ends with a barrier.
template <bool kLds>
__device__ __forceinline__ LogitRows<kLds> router_contract_f32(
    const float *__restrict__ x, const float *__restrict__ w_r, const float *__restrict__ bias, int64_t T, int d,
    int N, float *__restrict__ logits_g, int64_t blk, float *s_lg, float (*s_x)[65]) {
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
  constexpr int kPer = kRouterTokens * kRouterChunk / kRouterThreads;  // pairs per thread
  for (int c0 = 0; c0 < N; c0 += kRouterChunk) {
    float acc[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) acc[q] = 0.f;
    for (int k0 = 0; k0 < d; k0 += kKc) {
      __syncthreads();
      for (int i = tid; i < kRouterTokens * kKc; i += kRouterThreads) {
        int t = i / kKc, k = i % kKc;
        s_x[t][k] = (t < nt && k0 + k < d) ? x[(t0 + t) * d + k0 + k] : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int pair = tid + q * kRouterThreads;
        const int t = pair / kRouterChunk, j = c0 + pair % kRouterChunk;
        if (j < N) {
          const float *w = w_r + (int64_t)j * d + k0;
          const int kn = min(kKc, d - k0);
          float a = acc[q];
          for (int k = 0; k < kn; ++k) a = __builtin_fmaf(s_x[t][k], w[k], a);
          acc[q] = a;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int pair = tid + q * kRouterThreads;
      const int t = pair / kRouterChunk, j = c0 + pair % kRouterChunk;
      if (j < N && t < nt) lg.at(t, kLds ? j - c0 : j) = acc[q] + (bias ? bias[j] : 0.f);
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
  __shared__ float s_max[kRouterTokens], s_inv[kRouterTokens];
  __shared__ int s_e[kRouterTokens], s_e2[kRouterTokens];
  const int64_t blk = blockIdx.x;
  const int64_t t0 = blk * kRouterTokens;
  const int nt = (int)min<int64_t>(kRouterTokens, T - t0);
  const LogitRows<kLds> lg = router_contract_f32<kLds>(x, w_r, bias, T, d, N, logits_g, blk, s_lg, s_x);
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
__device__ void router_bwd_epilogue(const LogitRows<kLds> lg, int nt, int64_t t0, const RouterBwdArgs &a,
                                    float *s_extra) {
  constexpr int kLpt = kThreads / kRouterTokens;  // lanes per token
  constexpr int kW = kThreads / kWave;
  const int N = a.N, d = a.d;
  const int tid = threadIdx.x, t = tid / kLpt, q = tid % kLpt;
  const float caux = a.d_aux * (float)N / ((float)a.T * (float)a.T);
  float *s_aux = s_extra;                // [kRouterChunk] (N <= kRouterChunk)
  float *s_wr = s_extra + kRouterChunk;  // [kW][kRouterChunk][kBwdWrCols]
  if (kLds) {
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
    for (int j = q; j < N; j += kLpt) sum += __expf(lg.at(t, j) - mx);
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
      const float pj = __expf(lg.at(t, j) - mx) * inv;
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
  for (int j = tid; j < N; j += kThreads) {
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

template <bool kLds>
__global__ __launch_bounds__(kRBThreads) void router_bwd_bf16_kernel(const RouterBwdArgs a) {
  __shared__ RouterSmem sm;
  const int64_t blk = blockIdx.x, t0 = blk * kRouterTokens;
  const int nt = (int)min<int64_t>(kRouterTokens, a.T - t0);
  const LogitRows<kLds> lg =
      router_contract_bf16<kLds>((const bf16 *)a.x, a.w_r, a.bias, a.T, a.d, a.N, a.logits, blk, sm);
  static_assert(kRouterTokens * (kRouterChunk + 1) + bwd_lds_floats<kRBThreads>() <= kRouterSmem / 4,
                "logit rows + backward scratch fit the staging area");
  router_bwd_epilogue<bf16, kRBThreads, kLds, false>(lg, nt, t0, a,
                                              (float *)sm.stage + kRouterTokens * (kRouterChunk + 1));
}

template <bool kLds>
__global__ __launch_bounds__(kRouterThreads) void router_bwd_f32_kernel(const RouterBwdArgs a) {
  __shared__ float s_lg[kLds ? kRouterTokens * (kRouterChunk + 1) : 1];
  __shared__ float s_x[kRouterTokens][65];
  const int64_t blk = blockIdx.x, t0 = blk * kRouterTokens;
  const int nt = (int)min<int64_t>(kRouterTokens, a.T - t0);
  const LogitRows<kLds> lg =
      router_contract_f32<kLds>((const float *)a.x, a.w_r, a.bias, a.T, a.d, a.N, a.logits, blk, s_lg, s_x);
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
    if (a.dtype == kBF16)
      (lds ? router_bwd_bf16_kernel<true> : router_bwd_bf16_kernel<false>)<<<dim3((unsigned)nb), dim3(kRBThreads), 0,
                                                                              st>>>(a);
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
    auto kern = lds ? router_bf16_kernel<true, kK> : router_bf16_kernel<false, kK>;
    kern<<<grid, dim3(kRBThreads), 0, st>>>((const bf16 *)a.x, a.w_r, a.bias, a.T, a.d, a.N, a.logits,
                                            a.expert_idx, a.gate, a.rank, a.bcount, a.ppart);
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
// Visibility across the XCDs without cache maintenance: every row is written
// once per launch with device-coherent (write-through) stores, which complete
// before the state word that announces them is stored; states are read with
// device-coherent loads; a row is read with ordinary cached loads only after
// its state was seen, so no cache can hold an older copy of it (rows are
// padded to 256 bytes, so no cache line spans two of them, and caches start
// each launch clean).  Counts are integers and P sums 2^-31 fixed-point
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

template <typename V>
__device__ __forceinline__ void store_through(V *p, V v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
__host__ __device__ constexpr int fused_tail_bytes(int N) { return N * 24 + kRouterTokens * 4 + 16 * 8 + 16; }
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
__device__ int lookback_window(const int32_t *state, int64_t lo, int32_t *err, bool &found) {
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
__device__ void route_fused_tail(const FusedRouteArgs &a, int64_t blk, int64_t nb, int nt, const int *s_e,
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
      store_through(rc + e, L.c[e]);
      store_through(rp + e, L.p[e]);
      L.xc[e] = 0;
      L.xp[e] = 0;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // this thread's stores are complete
  __syncthreads();
  if (tid == 0) __hip_atomic_store(state + blk, blk == 0 ? 2 : 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

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
      store_through(a.inc_c + blk * Ns + e, L.xc[e] + L.c[e]);
      store_through(a.inc_p + blk * Ns + e, L.xp[e] + L.p[e]);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) __hip_atomic_store(state + blk, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
__global__ __launch_bounds__(kRBThreads) void route_fused_bf16_kernel(const FusedRouteArgs a) {
  static_assert(kRouterLgBytes + fused_tail_bytes(kFusedMaxExperts) <= kRouterSmem, "tail LDS");
  __shared__ RouterSmem sm;
  __shared__ int s_blk;
  const int64_t T = a.r.T, nb = router_blocks(T);
  const int64_t blk = route_ticket(a.sync, &s_blk);
  if (blk >= nb) return;
  const int N = a.r.N;
  const LogitRows<kLds> lg =
      router_contract_bf16<kLds>((const bf16 *)a.r.x, a.r.w_r, a.r.bias, T, a.r.d, N, a.r.logits, blk, sm);
  const int64_t t0 = blk * kRouterTokens;
  const int nt = (int)min<int64_t>(kRouterTokens, T - t0);
  const TailLds L = tail_lds(sm.stage + kRouterLgBytes, N);
  router_epilogue<kRBThreads, kLds, 1>(lg, nt, N, t0, blk, TopK{T, nb}, a.r.expert_idx, a.r.gate, a.r.slot,
                                       a.r.bcount, a.r.ppart, sm.s_max, sm.s_inv, sm.s_e, sm.s_e2, L.c, L.p);
  route_fused_tail<kRBThreads>(a, blk, nb, nt, sm.s_e, L);
}

template <bool kLds>
__global__ __launch_bounds__(kRouterThreads) void route_fused_f32_kernel(const FusedRouteArgs a) {
  constexpr int kLg = kLds ? kRouterTokens * (kRouterChunk + 1) * 4 : 0;
  constexpr int kX = kRouterTokens * 65 * 4;
  constexpr int kTail = fused_tail_bytes(kFusedMaxExperts);
  __shared__ __attribute__((aligned(16))) char s_buf[kLg + (kX > kTail ? kX : kTail)];
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
                                                       (float(*)[65])(s_buf + kLg));
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
      auto kern = lds ? route_fused_bf16_kernel<true> : route_fused_bf16_kernel<false>;
      kern<<<dim3((unsigned)nb), dim3(kRBThreads), 0, st>>>(a);
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
