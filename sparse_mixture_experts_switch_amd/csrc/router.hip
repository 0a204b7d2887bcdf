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
// significant bits), so every product x_k * plane_k is exact in fp32 and the
// fp32 accumulation sees the same terms as an fp32 dot product.
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
// block's tokens, from logits already complete in `lg`.
template <bool kLds>
__device__ void router_epilogue(const LogitRows<kLds> lg, int nt, int N, int64_t t0, int64_t blk,
                                int32_t *__restrict__ expert_idx, float *__restrict__ gate,
                                int32_t *__restrict__ slot_rank, int32_t *__restrict__ bcount,
                                float *__restrict__ ppart, float *s_max, float *s_inv, int *s_e) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  constexpr int kWaves = kRouterThreads / kWave;
  for (int t = wave; t < nt; t += kWaves) {
    float best = -INFINITY;
    int bi = 0x7fffffff;
    for (int j = lane; j < N; j += kWave) {
      float h = lg.at(t, j);
      if (h > best) {  // ascending j per lane: first maximum kept
        best = h;
        bi = j;
      }
    }
    wave_argmax(best, bi);
    float s = 0.f;
    for (int j = lane; j < N; j += kWave) s += __expf(lg.at(t, j) - best);
    s = wave_sum(s);
    if (lane == 0) {
      float inv = 1.0f / s;
      s_max[t] = best;
      s_inv[t] = inv;
      s_e[t] = bi;
      expert_idx[t0 + t] = bi;
      gate[t0 + t] = inv;  // p_e = exp(h_e - max) / s with h_e = max
    }
  }
  __syncthreads();
  for (int j = tid; j < N; j += kRouterThreads) {
    float p = 0.f;
    int c = 0;
    for (int t = 0; t < nt; ++t) {
      p += __expf(lg.at(t, j) - s_max[t]) * s_inv[t];
      c += (s_e[t] == j);
    }
    ppart[blk * N + j] = p;
    bcount[blk * N + j] = c;
  }
  for (int t = tid; t < nt; t += kRouterThreads) {
    int e = s_e[t], r = 0;
    for (int u = 0; u < t; ++u) r += (s_e[u] == e);
    slot_rank[t0 + t] = r;
  }
}

// ---------------------------------------------------------------------------
// bf16 activations, 3-plane bf16 MFMA (v_mfma_f32_16x16x32_bf16).
// Wave w computes experts [c0 + 32w, c0 + 32w + 32) for all 32 tokens of the
// block: 2 token tiles x 2 expert tiles of 16x16.
// MFMA operand layout (16x16x32): lane l supplies row (l % 16) and the 8
// consecutive k values starting at 8 * (l / 16); the result lane l holds
// column (l % 16), rows 4 * (l / 16) + i.
// ---------------------------------------------------------------------------
template <bool kLds>
__global__ __launch_bounds__(kRouterThreads) void router_bf16_kernel(
    const bf16 *__restrict__ x, const float *__restrict__ w_r, const float *__restrict__ bias,
    int64_t T, int d, int N, float *__restrict__ logits_g, int32_t *__restrict__ expert_idx,
    float *__restrict__ gate, int32_t *__restrict__ slot_rank, int32_t *__restrict__ bcount,
    float *__restrict__ ppart) {
  static_assert(kRouterTokens == 32 && kRouterThreads == 256, "tile shape");
  __shared__ float s_lg[kLds ? kRouterTokens * (kRouterChunk + 1) : 1];
  __shared__ float s_max[kRouterTokens], s_inv[kRouterTokens];
  __shared__ int s_e[kRouterTokens];

  const int64_t blk = blockIdx.x;
  const int64_t t0 = blk * kRouterTokens;
  const int nt = (int)min<int64_t>(kRouterTokens, T - t0);
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int r16 = lane % 16, kq = (lane / 16) * 8;

  LogitRows<kLds> lg;
  if (kLds) {
    lg.base = s_lg;
    lg.stride = kRouterChunk + 1;
  } else {
    lg.base = logits_g + t0 * N;
    lg.stride = N;
  }

  // token rows this lane feeds to the A operand (clamped inside the batch)
  const int64_t ta0 = t0 + min(r16, nt - 1);
  const int64_t ta1 = t0 + min(16 + r16, nt - 1);
  const bf16 *xa0 = x + ta0 * d + kq;
  const bf16 *xa1 = x + ta1 * d + kq;

  for (int c0 = 0; c0 < N; c0 += kRouterChunk) {
    const int e0 = c0 + wave * 32 + r16;  // expert of B tile 0 for this lane
    const int e1 = e0 + 16;
    const bool v0 = e0 < N, v1 = e1 < N;
    const float *wb0 = w_r + (int64_t)(v0 ? e0 : 0) * d + kq;
    const float *wb1 = w_r + (int64_t)(v1 ? e1 : 0) * d + kq;
    f32x4 acc[2][2] = {};
    if (c0 + wave * 32 < N) {
      for (int k = 0; k < d; k += 32) {
        bf16x8 a0 = as_bf16x8(*(const u32x4 *)(xa0 + k));
        bf16x8 a1 = as_bf16x8(*(const u32x4 *)(xa1 + k));
        bf16x8 bh[2], bm[2], bl[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const float *wp = (q == 0 ? wb0 : wb1) + k;
          const bool valid = q == 0 ? v0 : v1;
          f32x4 w0 = *(const f32x4 *)wp;
          f32x4 w1 = *(const f32x4 *)(wp + 4);
          if (!valid) {
            w0 = f32x4{0.f, 0.f, 0.f, 0.f};
            w1 = w0;
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            bf16 h, m, l;
            split3(i < 4 ? w0[i] : w1[i - 4], h, m, l);
            bh[q][i] = h;
            bm[q][i] = m;
            bl[q][i] = l;
          }
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          acc[0][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bh[q], acc[0][q], 0, 0, 0);
          acc[1][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bh[q], acc[1][q], 0, 0, 0);
          acc[0][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bm[q], acc[0][q], 0, 0, 0);
          acc[1][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bm[q], acc[1][q], 0, 0, 0);
          acc[0][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bl[q], acc[0][q], 0, 0, 0);
          acc[1][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bl[q], acc[1][q], 0, 0, 0);
        }
      }
    }
    // scatter the 32 x 32 logits tile of this wave
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int j = c0 + wave * 32 + q * 16 + r16;
        if (j < N) {
          const float b = bias ? bias[j] : 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = tb * 16 + (lane / 16) * 4 + i;
            if (t < nt) lg.at(t, kLds ? j - c0 + 0 : j) = acc[tb][q][i] + b;
          }
        }
      }
    if (kLds) break;  // N <= kRouterChunk: one chunk holds every expert
  }
  __syncthreads();
  router_epilogue<kLds>(lg, nt, N, t0, blk, expert_idx, gate, slot_rank, bcount, ppart, s_max, s_inv,
                        s_e);
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
    if (lds)
      router_bf16_kernel<true><<<grid, block, 0, st>>>((const bf16 *)a.x, a.w_r, a.bias, a.T, a.d, a.N,
                                                       a.logits, a.expert_idx, a.gate, a.slot, a.bcount,
                                                       a.ppart);
    else
      router_bf16_kernel<false><<<grid, block, 0, st>>>((const bf16 *)a.x, a.w_r, a.bias, a.T, a.d, a.N,
                                                        a.logits, a.expert_idx, a.gate, a.slot, a.bcount,
                                                        a.ppart);
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
