// Capacity assignment and the load-balancing loss.
//
// Switch Transformers write-up, "Expert Capacity and the Capacity Factor":
// every expert has a buffer of `capacity` tokens and the tokens that overflow
// it are dropped.  Overflow is decided in token order: a token's slot is the
// number of earlier tokens of the batch routed to the same expert, and the
// token is dropped when that number reaches the capacity.  "The Load-Balancing
// Loss": loss = N * sum_i f_i P_i with f_i the fraction of tokens whose argmax
// is expert i and P_i the batch mean of p_i(x).
//
// The router leaves, per block of kRouterTokens tokens, the block's count for
// every expert (bcount[b][i]) and every token's rank inside its block.  The
// scan turns bcount into exclusive offsets over blocks, in place, with integer
// arithmetic only, so slots and drops are exact and independent of scheduling.

#include "common.h"
#include "launch.h"

namespace smx {

constexpr int kScanWaves = 16;

// One workgroup per 64 experts (lane = expert).  Wave w owns a contiguous
// segment of blocks: it sums its segment, the segment sums are scanned in LDS,
// then the wave rewrites its segment as exclusive offsets.  The P partial sums
// are reduced in the same fixed order (segment by segment).  Loads are issued
// kScanBatch at a time so that each wave waits for memory once per batch, not
// once per block.
constexpr int kScanBatch = 8;

__global__ __launch_bounds__(kScanWaves *kWave) void assign_scan_kernel(
    int32_t *__restrict__ bcount, const float *__restrict__ ppart, int64_t nb, int N,
    int32_t *__restrict__ expert_count, float *__restrict__ psum) {
  __shared__ int s_cnt[kScanWaves][kWave];
  __shared__ float s_p[kScanWaves][kWave];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int j = blockIdx.x * kWave + lane;
  const bool valid = j < N;
  const int jj = valid ? j : N - 1;  // lanes past N read a valid column
  const int64_t seg = ceil_div(nb, kScanWaves);
  const int64_t b0 = min<int64_t>(nb, wave * seg), b1 = min<int64_t>(nb, b0 + seg);
  int c = 0;
  float p = 0.f;
  for (int64_t b = b0; b < b1; b += kScanBatch) {
    int cv[kScanBatch];
    float pv[kScanBatch];
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i) {
      const int64_t bb = min(b + i, b1 - 1);
      cv[i] = bcount[bb * N + jj];
      pv[i] = ppart[bb * N + jj];
    }
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i)
      if (b + i < b1) {
        c += cv[i];
        p += pv[i];
      }
  }
  s_cnt[wave][lane] = c;
  s_p[wave][lane] = p;
  __syncthreads();
  int run = 0;
  for (int w = 0; w < wave; ++w) run += s_cnt[w][lane];
  for (int64_t b = b0; b < b1; b += kScanBatch) {
    int cv[kScanBatch];
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i) cv[i] = bcount[min(b + i, b1 - 1) * N + jj];
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i)
      if (b + i < b1) {
        if (valid) bcount[(b + i) * N + j] = run;
        run += cv[i];
      }
  }
  if (wave == 0 && valid) {
    int tot = 0;
    float ps = 0.f;
    for (int w = 0; w < kScanWaves; ++w) {
      tot += s_cnt[w][lane];
      ps += s_p[w][lane];
    }
    expert_count[j] = tot;
    psum[j] = ps;
  }
}

// N * sum_i (count_i / T) (psum_i / T) by one 256-thread block, reduced in
// double in a fixed order.
__device__ void write_aux_loss(int64_t T, int N, const int32_t *__restrict__ expert_count,
                               const float *__restrict__ psum, float *__restrict__ aux_loss) {
  __shared__ double s_acc[256];
  double acc = 0.0;
  for (int j = threadIdx.x; j < N; j += 256) acc += (double)expert_count[j] * (double)psum[j];
  s_acc[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) s_acc[threadIdx.x] += s_acc[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double tt = (double)T;
    aux_loss[0] = T > 0 ? (float)(s_acc[0] * (double)N / (tt * tt)) : 0.f;
  }
}

// slot = in-block rank + the block's offset for the token's expert;
// dropped = slot >= capacity.  Block 0 also forms the loss.
__global__ __launch_bounds__(256) void assign_apply_kernel(
    const int32_t *__restrict__ expert_idx, int32_t *__restrict__ slot, uint8_t *__restrict__ dropped,
    const int32_t *__restrict__ boff, int64_t T, int N, int C, const int32_t *__restrict__ expert_count,
    const float *__restrict__ psum, float *__restrict__ aux_loss) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t < T) {
    const int e = expert_idx[t];
    const int s = slot[t] + boff[(t / kRouterTokens) * N + e];
    slot[t] = s;
    dropped[t] = s >= C ? 1 : 0;
  }
  if (blockIdx.x == 0) write_aux_loss(T, N, expert_count, psum, aux_loss);
}

// Layer path variant of the apply step: besides slot and dropped it records
// which token sits in each live slot (tok[e][slot] = t) and its gate
// (gmap[e][slot]) for the expert FFN to gather from and scatter to, and
// writes the output rows of dropped tokens (their computation is skipped: 0,
// or x when a residual is added).
__global__ __launch_bounds__(256) void assign_apply_layer_kernel(
    const int32_t *__restrict__ expert_idx, int32_t *__restrict__ slot, uint8_t *__restrict__ dropped,
    const int32_t *__restrict__ boff, int64_t T, int N, int C, const int32_t *__restrict__ expert_count,
    const float *__restrict__ psum, float *__restrict__ aux_loss, int32_t *__restrict__ tok,
    float *__restrict__ gmap, const float *__restrict__ gate, const u32x4 *__restrict__ xres,
    u32x4 *__restrict__ y, int row16) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int lane = threadIdx.x % kWave;
  bool drop = false;
  if (t < T) {
    const int e = expert_idx[t];
    const int s = slot[t] + boff[(t / kRouterTokens) * N + e];
    slot[t] = s;
    drop = s >= C;
    dropped[t] = drop ? 1 : 0;
    if (!drop) {
      tok[(int64_t)e * C + s] = (int32_t)t;
      gmap[(int64_t)e * C + s] = gate[t];
    }
  }
  unsigned long long mask = __ballot(drop);
  while (mask) {
    const int b = __ffsll(mask) - 1;
    mask &= mask - 1;
    const int64_t tt = t - lane + b;
    for (int c = lane; c < row16; c += kWave) y[tt * row16 + c] = xres ? xres[tt * row16 + c] : u32x4{0, 0, 0, 0};
  }
  if (blockIdx.x == 0) write_aux_loss(T, N, expert_count, psum, aux_loss);
}

// Empty batch: every count is 0 and the loss is 0.
__global__ void route_empty_kernel(int N, int32_t *__restrict__ expert_count, float *__restrict__ aux_loss) {
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < N; j += gridDim.x * blockDim.x) expert_count[j] = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) aux_loss[0] = 0.f;
}

hipError_t launch_assign_scan(const RouteArgs &a, hipStream_t st) {
  const int64_t nb = router_blocks(a.T);
  if (nb == 0) {
    route_empty_kernel<<<dim3((unsigned)ceil_div(a.N, 256)), dim3(256), 0, st>>>(a.N, a.expert_count, a.aux_loss);
    return hipGetLastError();
  }
  assign_scan_kernel<<<dim3((unsigned)ceil_div(a.N, kWave)), dim3(kScanWaves * kWave), 0, st>>>(
      a.bcount, a.ppart, nb, a.N, a.expert_count, a.psum);
  return hipGetLastError();
}

hipError_t launch_assign_apply(const RouteArgs &a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  assign_apply_kernel<<<dim3((unsigned)ceil_div(a.T, 256)), dim3(256), 0, st>>>(
      a.expert_idx, a.slot, a.dropped, a.bcount, a.T, a.N, a.C, a.expert_count, a.psum, a.aux_loss);
  return hipGetLastError();
}

hipError_t launch_assign_apply_layer(const RouteArgs &a, int32_t *tok, float *gmap, const void *xres, void *y,
                                     hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  const int row16 = a.d * (a.dtype == kBF16 ? 2 : 4) / 16;
  assign_apply_layer_kernel<<<dim3((unsigned)ceil_div(a.T, 256)), dim3(256), 0, st>>>(
      a.expert_idx, a.slot, a.dropped, a.bcount, a.T, a.N, a.C, a.expert_count, a.psum, a.aux_loss, tok, gmap,
      a.gate, (const u32x4 *)xres, (u32x4 *)y, row16);
  return hipGetLastError();
}

}  // namespace smx
