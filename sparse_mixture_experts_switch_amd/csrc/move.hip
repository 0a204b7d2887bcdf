// Dispatch (gather into per-expert buffers) and combine (gate-scaled scatter
// back to token order).
//
// Switch Transformers write-up: the figure of "Expert Capacity and the
// Capacity Factor" (dispatch each token to its single top expert, overflow
// beyond capacity goes to the residual, combine scales each output by the gate
// p_i(x)), and the combine equation y = sum_{i in T} p_i(x) E_i(x) of "Switch
// Routing" with k = 1.  A dropped token's computation is skipped: its bare
// output is 0, and with the residual it is x.
//
// Both kernels move whole rows with 16-byte vector accesses, one wave per
// token; they are bound by HBM bandwidth.
//
// The block's Add + Normalize after the layer (the architecture figure of
// "The Architecture in Place") is here too: layer normalisation over d_model
// of x + y, one wave per row.

#include "common.h"
#include "launch.h"

namespace smx {

constexpr int kMoveThreads = 256;
constexpr int kMoveTokens = kMoveThreads / kWave;  // one wave per token

__global__ __launch_bounds__(kMoveThreads) void dispatch_kernel(
    const u32x4 *__restrict__ x, const int32_t *__restrict__ expert_idx, const int32_t *__restrict__ slot,
    const uint8_t *__restrict__ dropped, u32x4 *__restrict__ out, int64_t T, int row16, int C) {
  const int64_t t = (int64_t)blockIdx.x * kMoveTokens + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (t >= T || dropped[t]) return;
  const u32x4 *src = x + t * row16;
  u32x4 *dst = out + ((int64_t)expert_idx[t] * C + slot[t]) * row16;
  for (int c = lane; c < row16; c += kWave) dst[c] = src[c];
}

template <typename T_>
__device__ __forceinline__ void combine_chunk(u32x4 &out, const u32x4 *eo, const u32x4 *xr, float g,
                                              bool keep);

template <>
__device__ __forceinline__ void combine_chunk<bf16>(u32x4 &out, const u32x4 *eo, const u32x4 *xr, float g,
                                                    bool keep) {
  bf16x8 r;
  bf16x8 e = keep ? as_bf16x8(*eo) : bf16x8{};
  bf16x8 xv = xr ? as_bf16x8(*xr) : bf16x8{};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float v = keep ? g * (float)e[i] : 0.f;
    if (xr) v = (float)xv[i] + v;
    r[i] = (bf16)v;
  }
  out = as_u32x4(r);
}

template <>
__device__ __forceinline__ void combine_chunk<float>(u32x4 &out, const u32x4 *eo, const u32x4 *xr, float g,
                                                     bool keep) {
  f32x4 e = keep ? __builtin_bit_cast(f32x4, *eo) : f32x4{};
  f32x4 xv = xr ? __builtin_bit_cast(f32x4, *xr) : f32x4{};
  f32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v = keep ? g * e[i] : 0.f;
    if (xr) v = xv[i] + v;
    r[i] = v;
  }
  out = __builtin_bit_cast(u32x4, r);
}

template <typename T_>
__global__ __launch_bounds__(kMoveThreads) void combine_kernel(
    const u32x4 *__restrict__ expert_out, const int32_t *__restrict__ expert_idx,
    const int32_t *__restrict__ slot, const uint8_t *__restrict__ dropped, const float *__restrict__ gate,
    const u32x4 *__restrict__ xres, u32x4 *__restrict__ y, int64_t T, int row16, int C) {
  const int64_t t = (int64_t)blockIdx.x * kMoveTokens + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (t >= T) return;
  const bool keep = !dropped[t];
  const float g = keep ? gate[t] : 0.f;
  const u32x4 *eo = keep ? expert_out + ((int64_t)expert_idx[t] * C + slot[t]) * row16 : nullptr;
  const u32x4 *xr = xres ? xres + t * row16 : nullptr;
  u32x4 *dst = y + t * row16;
  for (int c = lane; c < row16; c += kWave) {
    u32x4 o;
    combine_chunk<T_>(o, keep ? eo + c : nullptr, xr ? xr + c : nullptr, g, keep);
    dst[c] = o;
  }
}

static inline int esize(int dtype) { return dtype == kBF16 ? 2 : 4; }

// out[t] = (v - mean v) / sqrt(var v + eps) * gamma + beta, v = x[t] + y[t]
// (x may be null), in fp32: the row stays in registers (P pieces of 16 bytes
// per lane), the mean and then the sum of squared deviations are each summed
// per lane in order and across the wave by fixed-order butterflies, so every
// run gives the same bits.  One rounding to the output type.
// With kCombine the row y[t] is the combine of the layer's stage API instead
// of a dense row: gate[t] * expert_out[expert_idx[t]][slot[t]] for a kept
// token, 0 for a dropped one, so that the block's output LayerNorm(x + y)
// is formed from the expert output in one pass (fp32 throughout, one
// rounding).
template <typename T_, int P, bool kCombine>
__global__ __launch_bounds__(kMoveThreads) void add_norm_kernel(const u32x4 *__restrict__ x, const u32x4 *y,
                                                               const float *__restrict__ gamma,
                                                               const float *__restrict__ beta, float eps,
                                                               u32x4 *out, int64_t T, int d, CombineRows cr) {
  constexpr int kE = 16 / sizeof(T_);  // values per 16-byte piece
  const int64_t t = (int64_t)blockIdx.x * kMoveTokens + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (t >= T) return;
  const int pieces = d / kE;
  bool keep = true;
  float g = 1.f;
  const u32x4 *yrow = y + t * pieces;
  if (kCombine) {
    keep = !cr.dropped[t];
    g = keep ? cr.gate[t] : 0.f;
    yrow = y + (keep ? (int64_t)cr.expert_idx[t] * cr.C + cr.slot[t] : 0) * pieces;
  }
  float v[P][kE];
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int c = lane + i * kWave;
    const bool in = c < pieces;
    const int cc = in ? c : 0;
    const u32x4 yv = keep ? yrow[cc] : u32x4{0, 0, 0, 0};
    const u32x4 xv = x ? x[t * pieces + cc] : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < kE; ++k) {
      float a, b;
      if constexpr (sizeof(T_) == 2) {
        a = (float)as_bf16x8(yv)[k];
        b = (float)as_bf16x8(xv)[k];
      } else {
        a = __builtin_bit_cast(f32x4, yv)[k];
        b = __builtin_bit_cast(f32x4, xv)[k];
      }
      v[i][k] = in ? (kCombine ? b + g * a : a + b) : 0.f;
      sum += v[i][k];
    }
  }
  const float mean = wave_sum(sum) / (float)d;
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < P; ++i)
    if (lane + i * kWave < pieces) {
#pragma unroll
      for (int k = 0; k < kE; ++k) {
        const float dv = v[i][k] - mean;
        sq += dv * dv;
      }
    }
  const float rstd = 1.0f / sqrtf(wave_sum(sq) / (float)d + eps);
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int c = lane + i * kWave;
    if (c >= pieces) continue;
    u32x4 o;
    if constexpr (sizeof(T_) == 2) {
      bf16x8 r;
#pragma unroll
      for (int k = 0; k < kE; ++k) r[k] = (bf16)((v[i][k] - mean) * rstd * gamma[c * kE + k] + beta[c * kE + k]);
      o = as_u32x4(r);
    } else {
      f32x4 r;
#pragma unroll
      for (int k = 0; k < kE; ++k) r[k] = (v[i][k] - mean) * rstd * gamma[c * kE + k] + beta[c * kE + k];
      o = __builtin_bit_cast(u32x4, r);
    }
    out[t * pieces + c] = o;
  }
}

template <typename T_, int P>
hipError_t run_add_norm(const AddNormArgs &a, hipStream_t st) {
  const dim3 grid((unsigned)ceil_div(a.T, kMoveTokens)), block(kMoveThreads);
  if (a.rows.expert_idx)
    add_norm_kernel<T_, P, true><<<grid, block, 0, st>>>((const u32x4 *)a.x, (const u32x4 *)a.y, a.gamma, a.beta,
                                                         a.eps, (u32x4 *)a.out, a.T, a.d, a.rows);
  else
    add_norm_kernel<T_, P, false><<<grid, block, 0, st>>>((const u32x4 *)a.x, (const u32x4 *)a.y, a.gamma,
                                                          a.beta, a.eps, (u32x4 *)a.out, a.T, a.d, a.rows);
  return hipGetLastError();
}

template <typename T_>
hipError_t add_norm_dispatch(const AddNormArgs &a, hipStream_t st) {
  const int pieces = a.d / (16 / (int)sizeof(T_));
  const int per = (int)ceil_div(pieces, kWave);
  if (per <= 1) return run_add_norm<T_, 1>(a, st);
  if (per <= 2) return run_add_norm<T_, 2>(a, st);
  if (per <= 4) return run_add_norm<T_, 4>(a, st);
  if (per <= 8) return run_add_norm<T_, 8>(a, st);
  return hipErrorInvalidValue;
}

int add_norm_max_d(int dtype) { return 8 * kWave * (dtype == kBF16 ? 8 : 4); }

hipError_t launch_add_norm(const AddNormArgs &a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  return a.dtype == kBF16 ? add_norm_dispatch<bf16>(a, st) : add_norm_dispatch<float>(a, st);
}

// Top-k combine ("Switch Routing" combine equation: the output is the sum
// over the token's selected experts of p_i(x) E_i(x)).  The expert FFN has
// already written each kept route's gate-scaled output to its own row r * T +
// t of `routed`; this adds the kept routes of every token in route order (and
// x, with the residual) in fp32 and rounds once.  One thread per 16-byte
// piece of an output row, consecutive threads on consecutive pieces.
template <typename T_, int kK>
__global__ __launch_bounds__(kMoveThreads) void topk_sum_kernel(const u32x4 *__restrict__ routed,
                                                                const uint8_t *__restrict__ dropped,
                                                                const u32x4 *__restrict__ x, u32x4 *__restrict__ y,
                                                                int64_t T, int row16) {
  constexpr int kE = 16 / sizeof(T_);
  const int64_t i = (int64_t)blockIdx.x * kMoveThreads + threadIdx.x;
  if (i >= T * row16) return;
  const int64_t t = i / row16;
  const int c = (int)(i - t * row16);
  float v[kE];
#pragma unroll
  for (int q = 0; q < kE; ++q) v[q] = 0.f;
#pragma unroll
  for (int r = 0; r < kK; ++r) {
    const int64_t row = r * T + t;
    if (dropped[row]) continue;
    const u32x4 w = routed[row * row16 + c];
#pragma unroll
    for (int q = 0; q < kE; ++q) {
      if constexpr (sizeof(T_) == 2)
        v[q] += (float)as_bf16x8(w)[q];
      else
        v[q] += __builtin_bit_cast(f32x4, w)[q];
    }
  }
  if (x) {
    const u32x4 w = x[t * row16 + c];
#pragma unroll
    for (int q = 0; q < kE; ++q) {
      if constexpr (sizeof(T_) == 2)
        v[q] = (float)as_bf16x8(w)[q] + v[q];
      else
        v[q] = __builtin_bit_cast(f32x4, w)[q] + v[q];
    }
  }
  u32x4 o;
  if constexpr (sizeof(T_) == 2) {
    bf16x8 r;
#pragma unroll
    for (int q = 0; q < kE; ++q) r[q] = (bf16)v[q];
    o = as_u32x4(r);
  } else {
    o = __builtin_bit_cast(u32x4, f32x4{v[0], v[1], v[2], v[3]});
  }
  y[t * row16 + c] = o;
}

hipError_t launch_topk_sum(const TopkSumArgs &a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  if (a.k != 2) return hipErrorInvalidValue;
  const int row16 = a.d * esize(a.dtype) / 16;
  const dim3 grid((unsigned)ceil_div(a.T * row16, kMoveThreads)), block(kMoveThreads);
  if (a.dtype == kBF16)
    topk_sum_kernel<bf16, 2><<<grid, block, 0, st>>>((const u32x4 *)a.routed, a.dropped, (const u32x4 *)a.x,
                                                     (u32x4 *)a.y, a.T, row16);
  else
    topk_sum_kernel<float, 2><<<grid, block, 0, st>>>((const u32x4 *)a.routed, a.dropped, (const u32x4 *)a.x,
                                                      (u32x4 *)a.y, a.T, row16);
  return hipGetLastError();
}

hipError_t launch_dispatch(const DispatchArgs &a, hipStream_t st) {
  if (a.T == 0 || a.C == 0) return hipSuccess;
  const int row16 = a.d * esize(a.dtype) / 16;
  dispatch_kernel<<<dim3((unsigned)ceil_div(a.T, kMoveTokens)), dim3(kMoveThreads), 0, st>>>(
      (const u32x4 *)a.x, a.expert_idx, a.slot, a.dropped, (u32x4 *)a.dispatched, a.T, row16, a.C);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs &a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  const int row16 = a.d * esize(a.dtype) / 16;
  dim3 grid((unsigned)ceil_div(a.T, kMoveTokens)), block(kMoveThreads);
  if (a.dtype == kBF16)
    combine_kernel<bf16><<<grid, block, 0, st>>>((const u32x4 *)a.expert_out, a.expert_idx, a.slot, a.dropped,
                                                 a.gate, (const u32x4 *)a.x_residual, (u32x4 *)a.y, a.T, row16,
                                                 a.C);
  else
    combine_kernel<float><<<grid, block, 0, st>>>((const u32x4 *)a.expert_out, a.expert_idx, a.slot,
                                                  a.dropped, a.gate, (const u32x4 *)a.x_residual, (u32x4 *)a.y,
                                                  a.T, row16, a.C);
  return hipGetLastError();
}

}  // namespace smx
