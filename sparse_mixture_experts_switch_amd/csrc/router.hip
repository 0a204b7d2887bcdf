// Router of the Switch layer: logits h = W_r . x (+ b), fp32 softmax, top-1
// expert, gate p_e(x), and the per-block partial results that the capacity
// assignment and the load-balancing loss are built from.
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
// block's earlier tokens with the same expert (stored in slot[] and later
// offset by the cross-block scan).
//
// bf16 activations: the contraction runs on bf16 MFMA.  W_r (fp32) is split
// exactly into three bf16 planes hi + mid + lo (each plane takes the next 8
// significant bits; a small kernel does it once per call), so every product
// x_k * plane_k is exact in fp32 and the fp32 accumulation sees the same
// terms as an fp32 dot product.
// fp32 activations: plain fp32 FMA on the vector ALUs.

#include "common.h"
#include "launch.h"

namespace smx {

// Exact split of an fp32 value into three bf16 values whose sum is the value.
__device__ __forceinline__ void split3(float w, bf16 &hi, bf16 &mid, bf16 &lo) {
  hi = (bf16)w;
  float r1 = w - (float)hi;
  mid = (bf16)r1;
  float r2 = r1 - (float)mid;
  lo = (bf16)r2;
}

template <bool kLds>
struct LogitRows {
  float *base;      // LDS [kRouterTokens][stride] or global [T][N] (row t0)
  int64_t stride;
  __device__ __forceinline__ float &at(int t, int j) const { return base[(int64_t)t * stride + j]; }
};

// Softmax, argmax, gate, P partials, block counts and in-block ranks for the
// block's tokens, from logits already complete in `lg`.  Four consecutive
// lanes share a token: each scans every fourth expert, then two butterfly
// steps combine the four partial results in a fixed order.
template <bool kLds>
__device__ void router_epilogue(const LogitRows<kLds> lg, int nt, int N, int64_t t0, int64_t blk,
                                int32_t *__restrict__ expert_idx, float *__restrict__ gate,
                                int32_t *__restrict__ slot_rank, int32_t *__restrict__ bcount,
                                float *__restrict__ ppart, float *s_max, float *s_inv, int *s_e) {
  static_assert(kRouterThreads == 4 * kRouterTokens, "4 lanes per token");
  const int tid = threadIdx.x;
  const int t = tid / 4, q = tid % 4;
  if (t < nt) {
    float best = -INFINITY;
    int bi = 0x7fffffff;
    for (int j = q; j < N; j += 4) {
      const float h = lg.at(t, j);
      if (h > best) {  // ascending j: first maximum kept
        best = h;
        bi = j;
      }
    }
#pragma unroll
    for (int off = 1; off < 4; off <<= 1) {
      const float ov = __shfl_xor(best, off, kWave);
      const int oi = __shfl_xor(bi, off, kWave);
      if (ov > best || (ov == best && oi < bi)) {
        best = ov;
        bi = oi;
      }
    }
    float sum = 0.f;
    for (int j = q; j < N; j += 4) sum += __expf(lg.at(t, j) - best);
    sum += __shfl_xor(sum, 1, kWave);
    sum += __shfl_xor(sum, 2, kWave);
    if (q == 0) {
      const float inv = 1.0f / sum;
      s_max[t] = best;
      s_inv[t] = inv;
      s_e[t] = bi;
      expert_idx[t0 + t] = bi;
      gate[t0 + t] = inv;  // p_e = exp(h_e - max) / sum with h_e = max
    }
  }  // the four lanes of a token are always on the same side of t < nt
  __syncthreads();
  for (int j = tid; j < N; j += kRouterThreads) {
    float p = 0.f;
    int c = 0;
    for (int u = 0; u < nt; ++u) {
      p += __expf(lg.at(u, j) - s_max[u]) * s_inv[u];
      c += (s_e[u] == j);
    }
    ppart[blk * N + j] = p;
    bcount[blk * N + j] = c;
  }
  if (tid < nt) {
    const int e = s_e[tid];
    int r = 0;
    for (int u = 0; u < tid; ++u) r += (s_e[u] == e);
    slot_rank[t0 + tid] = r;
  }
}

// ---------------------------------------------------------------------------
// bf16 activations, 3-plane bf16 MFMA (v_mfma_f32_16x16x32_bf16).
// The block's 64 token rows and the 128-expert chunk of the three W_r planes
// move through LDS 64 contraction columns at a time: global loads are
// row-contiguous (8 lanes cover one 128-byte row piece, the access pattern
// the L1/L2 path serves fastest), a register ring keeps kRouterDepth chunks
// in flight, and the MFMA operands are then read from padded LDS rows.
// Wave w computes experts [c0 + 32w, c0 + 32w + 32) for all 64 tokens: 4
// token tiles x 2 expert tiles of 16x16, three planes each.
// MFMA operand layout (16x16x32): lane l supplies row (l % 16) and the 8
// consecutive k values starting at 8 * (l / 16); the result lane l holds
// column (l % 16), rows 4 * (l / 16) + i.
// ---------------------------------------------------------------------------
constexpr int kRouterDepth = 2;
constexpr int kTokTiles = kRouterTokens / 16;
constexpr int kRKC = 64;                     // contraction columns per chunk
constexpr int kRLS = kRKC + 8;               // padded LDS row (bf16)
constexpr int kXPer = kRouterTokens * (kRKC / 8) / kRouterThreads;      // 16-byte x pieces per thread
constexpr int kWPer = 3 * kRouterChunk * (kRKC / 8) / kRouterThreads;  // 16-byte plane pieces per thread
constexpr int kXStage = kRouterTokens * kRLS;                          // bf16 per x stage
constexpr int kWStage = 3 * kRouterChunk * kRLS;                       // bf16 per plane stage
constexpr int kRouterStageBytes = 2 * (kXStage + kWStage) * 2;
constexpr int kRouterLgBytes = kRouterTokens * (kRouterChunk + 1) * 4;
constexpr int kRouterSmem = kRouterStageBytes > kRouterLgBytes ? kRouterStageBytes : kRouterLgBytes;

template <bool kLds>
__global__ __launch_bounds__(kRouterThreads) void router_bf16_kernel(
    const bf16 *__restrict__ x, const bf16 *__restrict__ planes, const float *__restrict__ bias,
    int64_t T, int d, int N, float *__restrict__ logits_g, int32_t *__restrict__ expert_idx,
    float *__restrict__ gate, int32_t *__restrict__ slot_rank, int32_t *__restrict__ bcount,
    float *__restrict__ ppart) {
  static_assert(kRouterThreads == 256 && kRouterChunk == 128, "4 waves x 32 experts");
  static_assert(kXPer * kRouterThreads == kRouterTokens * (kRKC / 8), "x pieces");
  static_assert(kWPer * kRouterThreads == 3 * kRouterChunk * (kRKC / 8), "plane pieces");
  __shared__ __attribute__((aligned(16))) char smem[kRouterSmem];
  __shared__ float s_max[kRouterTokens], s_inv[kRouterTokens];
  __shared__ int s_e[kRouterTokens];
  bf16 *xs = (bf16 *)smem;              // [2][64][kRLS]
  bf16 *ws = xs + 2 * kXStage;          // [2][3][128][kRLS]

  const int64_t blk = blockIdx.x;
  const int64_t t0 = blk * kRouterTokens;
  const int nt = (int)min<int64_t>(kRouterTokens, T - t0);
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int r16 = lane % 16, kq = (lane / 16) * 8;
  const int64_t plane = (int64_t)N * d;
  const int nk = d / kRKC;

  LogitRows<kLds> lg;
  if (kLds) {
    lg.base = (float *)smem;  // reuses the staging buffers after the contraction
    lg.stride = kRouterChunk + 1;
  } else {
    lg.base = logits_g + t0 * N;
    lg.stride = N;
  }

  // Row-contiguous load plan: piece i covers 16 bytes of row i / 8.
  const bf16 *xsrc[kXPer];
  int xoff[kXPer];
#pragma unroll
  for (int q = 0; q < kXPer; ++q) {
    const int i = tid + q * kRouterThreads, r = i / 8, c = i % 8;
    xsrc[q] = x + (t0 + min(r, nt - 1)) * d + c * 8;
    xoff[q] = r * kRLS + c * 8;
  }

  for (int c0 = 0; c0 < N; c0 += kRouterChunk) {
    const bf16 *wsrc[kWPer];
    int woff[kWPer];
#pragma unroll
    for (int q = 0; q < kWPer; ++q) {
      const int i = tid + q * kRouterThreads, row = i / 8, c = i % 8;  // row = plane * 128 + expert
      const int pl = row / kRouterChunk, e = row % kRouterChunk;
      wsrc[q] = planes + pl * plane + (int64_t)min(c0 + e, N - 1) * d + c * 8;
      woff[q] = row * kRLS + c * 8;
    }
    u32x4 xr[kRouterDepth][kXPer], wr[kRouterDepth][kWPer];
    auto fetch = [&](int slot, int ch) {
      const int k0 = min(ch, nk - 1) * kRKC;
#pragma unroll
      for (int q = 0; q < kXPer; ++q) xr[slot][q] = *(const u32x4 *)(xsrc[q] + k0);
#pragma unroll
      for (int q = 0; q < kWPer; ++q) wr[slot][q] = *(const u32x4 *)(wsrc[q] + k0);
    };
    auto store = [&](int slot, int buf) {
#pragma unroll
      for (int q = 0; q < kXPer; ++q) *(u32x4 *)(xs + buf * kXStage + xoff[q]) = xr[slot][q];
#pragma unroll
      for (int q = 0; q < kWPer; ++q) *(u32x4 *)(ws + buf * kWStage + woff[q]) = wr[slot][q];
    };
    f32x4 acc[kTokTiles][2];
#pragma unroll
    for (int tb = 0; tb < kTokTiles; ++tb) acc[tb][0] = acc[tb][1] = f32x4{0.f, 0.f, 0.f, 0.f};

    __syncthreads();  // previous chunk's readers of the staging buffers are done
#pragma unroll
    for (int j = 0; j < kRouterDepth; ++j) fetch(j, j);
    store(0, 0);
    __syncthreads();
    for (int base = 0; base < nk; base += kRouterDepth) {
#pragma clang loop unroll(full)
      for (int j = 0; j < kRouterDepth; ++j) {
        const int ch = base + j;
        if (ch < nk) {
          const bf16 *xb = xs + (ch & 1) * kXStage;
          const bf16 *wbuf = ws + (ch & 1) * kWStage;
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            bf16x8 b[2][3];
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
              for (int pl = 0; pl < 3; ++pl)
                b[q][pl] = as_bf16x8(*(const u32x4 *)(
                    wbuf + (pl * kRouterChunk + wave * 32 + q * 16 + r16) * kRLS + s * 32 + kq));
#pragma unroll
            for (int tb = 0; tb < kTokTiles; ++tb) {
              const bf16x8 a = as_bf16x8(*(const u32x4 *)(xb + (tb * 16 + r16) * kRLS + s * 32 + kq));
#pragma unroll
              for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int pl = 0; pl < 3; ++pl)
                  acc[tb][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[q][pl], acc[tb][q], 0, 0, 0);
            }
          }
        }
        fetch(j, ch + kRouterDepth);
        store((j + 1) % kRouterDepth, (ch + 1) & 1);
        __syncthreads();
      }
    }
    // scatter this wave's 64 x 32 logits tile (the staging buffers are free:
    // the loop ended with a barrier)
#pragma unroll
    for (int tb = 0; tb < kTokTiles; ++tb)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int j = c0 + wave * 32 + q * 16 + r16;
        if (j < N) {
          const float b = bias ? bias[j] : 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = tb * 16 + (lane / 16) * 4 + i;
            if (t < nt) lg.at(t, kLds ? j - c0 : j) = acc[tb][q][i] + b;
          }
        }
      }
    if (kLds) break;  // N <= kRouterChunk: one chunk holds every expert
  }
  __syncthreads();
  router_epilogue<kLds>(lg, nt, N, t0, blk, expert_idx, gate, slot_rank, bcount, ppart, s_max, s_inv,
                        s_e);
}

// W_r split once per call into three bf16 planes [3][N][d] (hi, mid, lo),
// 8 values per thread.
__global__ __launch_bounds__(256) void router_split_kernel(const float *__restrict__ w_r, int64_t n8,
                                                           u32x4 *__restrict__ planes) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = ((const f32x4 *)w_r)[2 * i], b = ((const f32x4 *)w_r)[2 * i + 1];
  bf16x8 h, m, l;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    bf16 hh, mm, ll;
    split3(k < 4 ? a[k] : b[k - 4], hh, mm, ll);
    h[k] = hh;
    m[k] = mm;
    l[k] = ll;
  }
  planes[i] = as_u32x4(h);
  planes[n8 + i] = as_u32x4(m);
  planes[2 * n8 + i] = as_u32x4(l);
}

// ---------------------------------------------------------------------------
// fp32 activations: fp32 FMA.  The block's x rows are staged in LDS in
// k-slices; each thread owns (token, expert) pairs of the current chunk.
// ---------------------------------------------------------------------------
template <bool kLds>
__global__ __launch_bounds__(kRouterThreads) void router_f32_kernel(
    const float *__restrict__ x, const float *__restrict__ w_r, const float *__restrict__ bias,
    int64_t T, int d, int N, float *__restrict__ logits_g, int32_t *__restrict__ expert_idx,
    float *__restrict__ gate, int32_t *__restrict__ slot_rank, int32_t *__restrict__ bcount,
    float *__restrict__ ppart) {
  constexpr int kK = 64;
  __shared__ float s_lg[kLds ? kRouterTokens * (kRouterChunk + 1) : 1];
  __shared__ float s_x[kRouterTokens][kK + 1];
  __shared__ float s_max[kRouterTokens], s_inv[kRouterTokens];
  __shared__ int s_e[kRouterTokens];

  const int64_t blk = blockIdx.x;
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
    for (int p = 0; p < kPer; ++p) acc[p] = 0.f;
    for (int k0 = 0; k0 < d; k0 += kK) {
      __syncthreads();
      for (int i = tid; i < kRouterTokens * kK; i += kRouterThreads) {
        int t = i / kK, k = i % kK;
        s_x[t][k] = (t < nt && k0 + k < d) ? x[(t0 + t) * d + k0 + k] : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int p = 0; p < kPer; ++p) {
        const int pair = tid + p * kRouterThreads;
        const int t = pair / kRouterChunk, j = c0 + pair % kRouterChunk;
        if (j < N) {
          const float *w = w_r + (int64_t)j * d + k0;
          const int kn = min(kK, d - k0);
          float a = acc[p];
          for (int k = 0; k < kn; ++k) a = __builtin_fmaf(s_x[t][k], w[k], a);
          acc[p] = a;
        }
      }
    }
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int pair = tid + p * kRouterThreads;
      const int t = pair / kRouterChunk, j = c0 + pair % kRouterChunk;
      if (j < N && t < nt) lg.at(t, kLds ? j - c0 : j) = acc[p] + (bias ? bias[j] : 0.f);
    }
    if (kLds) break;
  }
  __syncthreads();
  router_epilogue<kLds>(lg, nt, N, t0, blk, expert_idx, gate, slot_rank, bcount, ppart, s_max, s_inv,
                        s_e);
}

hipError_t launch_router(const RouteArgs &a, hipStream_t st) {
  const int64_t nb = ceil_div(a.T, kRouterTokens);
  if (nb == 0) return hipSuccess;
  const bool lds = a.N <= kRouterChunk;
  dim3 grid((unsigned)nb), block(kRouterThreads);
  if (a.dtype == kBF16) {
    const int64_t n8 = (int64_t)a.N * a.d / 8;
    router_split_kernel<<<dim3((unsigned)ceil_div(n8, 256)), dim3(256), 0, st>>>(a.w_r, n8, (u32x4 *)a.planes);
    if (lds)
      router_bf16_kernel<true><<<grid, block, 0, st>>>((const bf16 *)a.x, (const bf16 *)a.planes, a.bias, a.T,
                                                       a.d, a.N, a.logits, a.expert_idx, a.gate, a.slot,
                                                       a.bcount, a.ppart);
    else
      router_bf16_kernel<false><<<grid, block, 0, st>>>((const bf16 *)a.x, (const bf16 *)a.planes, a.bias, a.T,
                                                        a.d, a.N, a.logits, a.expert_idx, a.gate, a.slot,
                                                        a.bcount, a.ppart);
  } else {
    if (lds)
      router_f32_kernel<true><<<grid, block, 0, st>>>((const float *)a.x, a.w_r, a.bias, a.T, a.d, a.N,
                                                      a.logits, a.expert_idx, a.gate, a.slot, a.bcount,
                                                      a.ppart);
    else
      router_f32_kernel<false><<<grid, block, 0, st>>>((const float *)a.x, a.w_r, a.bias, a.T, a.d, a.N,
                                                       a.logits, a.expert_idx, a.gate, a.slot, a.bcount,
                                                       a.ppart);
  }
  return hipGetLastError();
}

}  // namespace smx
