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
// assignment turns the counts into exclusive offsets over blocks with integer
// arithmetic only, so slots and drops are exact and independent of
// scheduling.  No kernel here modifies its inputs: each one can be run again
// on the same buffers with the same result.

#include "common.h"
#include "launch.h"

namespace smx {

constexpr int kScanWaves = 16;

// Virtual token j = r * Tp + t (route r of token t, Tp a multiple of the
// router block): its token t and its index o = r * T + t in the per-route
// outputs; false past the batch.  k <= 2.
__device__ __forceinline__ bool virt_token(int64_t j, int64_t T, int64_t Tp, int k, int64_t &t, int64_t &o) {
  const int r = (k > 1 && j >= Tp) ? 1 : 0;
  t = j - r * Tp;
  o = r * T + t;
  return t < T;
}

// One workgroup per 64 experts (lane = expert).  Wave w owns a contiguous
// segment of blocks: it sums its segment, the segment sums are scanned in LDS,
// then the wave rewrites its segment as exclusive offsets.  The P partial sums
// are reduced in the same fixed order (segment by segment).  Loads are issued
// kScanBatch at a time so that each wave waits for memory once per batch, not
// once per block.
constexpr int kScanBatch = 8;

__global__ __launch_bounds__(kScanWaves *kWave) void assign_scan_kernel(
    const int32_t *__restrict__ bcount, int32_t *__restrict__ boff, const float *__restrict__ ppart, int64_t nb,
    int N, int32_t *__restrict__ expert_count, float *__restrict__ psum) {
  __shared__ int s_cnt[kScanWaves][kWave];
  __shared__ float s_p[kScanWaves][kWave];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int j = blockIdx.x * kWave + lane;
  const bool valid = j < N;
  const int jj = valid ? j : N - 1;  // lanes past N read a valid column
  const int64_t Np = count_stride(N);
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
      cv[i] = bcount[bb * Np + jj];
      pv[i] = ppart[bb * Np + jj];
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
    for (int i = 0; i < kScanBatch; ++i) cv[i] = bcount[min(b + i, b1 - 1) * Np + jj];
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i)
      if (b + i < b1) {
        if (valid) boff[(b + i) * Np + j] = run;
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

// N * sum_i (count_i / (k T)) (psum_i / T) by one 256-thread block, reduced
// in double in a fixed order.
__device__ void write_aux_loss(int64_t T, int k, int N, const int32_t *__restrict__ expert_count,
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
    aux_loss[0] = T > 0 ? (float)(s_acc[0] * (double)N / ((double)k * tt * tt)) : 0.f;
  }
}

// slot = in-block rank + the block's offset for the route's expert;
// dropped = slot >= capacity.  Block 0 also forms the loss.  One thread per
// virtual token.
__global__ __launch_bounds__(256) void assign_apply_kernel(
    const int32_t *__restrict__ expert_idx, const int32_t *__restrict__ rank, int32_t *__restrict__ slot,
    uint8_t *__restrict__ dropped,
    const int32_t *__restrict__ boff, int64_t T, int64_t Tp, int k, int N, int C,
    const int32_t *__restrict__ expert_count, const float *__restrict__ psum, float *__restrict__ aux_loss) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int64_t t, o;
  if (virt_token(j, T, Tp, k, t, o)) {
    const int e = expert_idx[o];
    const int s = rank[j] + boff[(j / kRouterTokens) * count_stride(N) + e];
    slot[o] = s;
    dropped[o] = s >= C ? 1 : 0;
  }
  if (blockIdx.x == 0) write_aux_loss(T, k, N, expert_count, psum, aux_loss);
}

// Output row of a dropped token whose layer output is 0, under the block's
// Add + Normalize ("The Architecture in Place"): (x - mean) / sqrt(var + eps)
// * gamma + beta over the row's d = 8 * row16 (bf16) or 4 * row16 (fp32)
// values, by one wave: per-lane partial sums in piece order, then fixed-order
// butterflies, so every run gives the same bits.  The row is read three
// times (sum, squared deviations, output); it is 16 * row16 bytes.
__device__ __forceinline__ void norm_row_wave(const u32x4 *__restrict__ xrow, u32x4 *__restrict__ orow, int row16,
                                              bool bf16_, const float *__restrict__ gamma,
                                              const float *__restrict__ beta, float eps, int lane) {
  const int per = bf16_ ? 8 : 4;
  const int d = row16 * per;
  auto val = [&](const u32x4 &v, int k) {
    return bf16_ ? (float)as_bf16x8(v)[k] : __builtin_bit_cast(f32x4, v)[k & 3];
  };
  float s = 0.f;
  for (int c = lane; c < row16; c += kWave) {
    const u32x4 v = xrow[c];
    for (int k = 0; k < per; ++k) s += val(v, k);
  }
  const float mean = wave_sum(s) / (float)d;
  float q = 0.f;
  for (int c = lane; c < row16; c += kWave) {
    const u32x4 v = xrow[c];
    for (int k = 0; k < per; ++k) {
      const float dv = val(v, k) - mean;
      q += dv * dv;
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum(q) / (float)d + eps);
  for (int c = lane; c < row16; c += kWave) {
    const u32x4 v = xrow[c];
    u32x4 o;
    if (bf16_) {
      bf16x8 r;
      for (int k = 0; k < 8; ++k) r[k] = (bf16)((val(v, k) - mean) * rstd * gamma[c * 8 + k] + beta[c * 8 + k]);
      o = as_u32x4(r);
    } else {
      f32x4 r;
      for (int k = 0; k < 4; ++k) r[k] = (val(v, k) - mean) * rstd * gamma[c * 4 + k] + beta[c * 4 + k];
      o = __builtin_bit_cast(u32x4, r);
    }
    orow[c] = o;
  }
}

// Layer path variant of the apply step: besides slot and dropped it records
// which token sits in each live slot (tok[e][slot] = t), the route's output
// row (rows[e][slot], when rows is set) and its gate (gmap[e][slot]) for the
// expert FFN to gather from and scatter to, and, when y is set (one route per
// token), writes the output rows of dropped tokens (their computation is
// skipped: 0, or x when a residual is added, or the Add + Normalize of x).
struct DropRows {
  const u32x4 *xres;
  u32x4 *y;
  int row16;
  bool bf16_;
  const float *gamma, *beta;  // set: normalized rows
  float eps;
};

__global__ __launch_bounds__(256) void assign_apply_layer_kernel(
    const int32_t *__restrict__ expert_idx, const int32_t *__restrict__ rank, int32_t *__restrict__ slot,
    uint8_t *__restrict__ dropped,
    const int32_t *__restrict__ boff, int64_t T, int64_t Tp, int k, int N, int C,
    const int32_t *__restrict__ expert_count, const float *__restrict__ psum, float *__restrict__ aux_loss,
    int32_t *__restrict__ tok, int32_t *__restrict__ rows, float *__restrict__ gmap, const float *__restrict__ gate,
    const DropRows dr) {
  const u32x4 *__restrict__ xres = dr.xres;
  u32x4 *__restrict__ y = dr.y;
  const int row16 = dr.row16;
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int lane = threadIdx.x % kWave;
  bool drop = false;
  int64_t t, o;
  if (virt_token(j, T, Tp, k, t, o)) {
    const int e = expert_idx[o];
    const int s = rank[j] + boff[(j / kRouterTokens) * count_stride(N) + e];
    slot[o] = s;
    drop = s >= C;
    dropped[o] = drop ? 1 : 0;
    if (!drop) {
      tok[(int64_t)e * C + s] = (int32_t)t;
      if (rows) rows[(int64_t)e * C + s] = (int32_t)o;
      gmap[(int64_t)e * C + s] = gate[o];
    }
  }
  if (y) {  // one route per token: virtual token = token
    unsigned long long mask = __ballot(drop);
    while (mask) {
      const int b = __ffsll(mask) - 1;
      mask &= mask - 1;
      const int64_t tt = j - lane + b;
      if (dr.gamma)
        norm_row_wave(xres + tt * row16, y + tt * row16, row16, dr.bf16_, dr.gamma, dr.beta, dr.eps, lane);
      else
        for (int c = lane; c < row16; c += kWave)
          y[tt * row16 + c] = xres ? xres[tt * row16 + c] : u32x4{0, 0, 0, 0};
    }
  }
  if (blockIdx.x == 0) write_aux_loss(T, k, N, expert_count, psum, aux_loss);
}

// Empty batch: every count is 0 and the loss is 0.
__global__ void route_empty_kernel(int N, int32_t *__restrict__ expert_count, float *__restrict__ aux_loss) {
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < N; j += gridDim.x * blockDim.x) expert_count[j] = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) aux_loss[0] = 0.f;
}

// ---------------------------------------------------------------------------
// One-launch assignment for batches whose block count is small.  Workgroup a
// owns router blocks [kAsBlocks a, kAsBlocks (a + 1)).  It sums the counts of
// all blocks before its own (16-byte loads, kAsBatch rows in flight per
// thread, 16 row groups, then the group sums in ascending order: exact
// integers), adds its own blocks' counts one by one for the offsets of each,
// and assigns its tokens.  One router block (64 tokens) per workgroup: the
// busiest workgroup reads the same prefix as with larger groups, and the
// token work (slots, maps, the rows of dropped tokens) spreads over four times
// the CUs (base workload 11.5 -> 10.3 us, large-shaped with 49% drops 21.5 ->
// 12.9 us, against four blocks per workgroup).  The workgroup holding the last block also reads the P
// partials of every block and forms the totals, the P sums and the loss.
// ---------------------------------------------------------------------------
constexpr int kAsThreads = 512;
constexpr int kAsBlocks = 1;                          // router blocks per workgroup
constexpr int kAsTokens = kAsBlocks * kRouterTokens;  // tokens per workgroup
constexpr int kAsGroups = kAsThreads / 32;            // row groups (32 lanes x 4 experts per row)
constexpr int kAsChunk = 128;                         // experts per pass
constexpr int kAsBatch = 16;

struct AssignArgs {
  const int32_t *expert_idx;
  const int32_t *rank;
  int32_t *slot;
  uint8_t *dropped;
  const int32_t *bcount;
  const float *ppart;
  int64_t T, Tp, nb;  // tokens, route stride of virtual tokens, blocks over all routes
  int k, N, C;
  int32_t *expert_count;
  float *psum, *aux_loss;
  const float *gate;
  int32_t *tok;   // layer path, or null
  int32_t *rows;  // layer path with k > 1, or null
  float *gmap;
  const u32x4 *xres;
  u32x4 *y;       // layer path with k = 1, or null
  int row16;
  bool bf16_;
  const float *gamma, *beta;  // set: dropped rows are the Add + Normalize of x
  float eps;
};

size_t assign_one_smem(int N) {
  return (size_t)kAsBlocks * N * 4 + (size_t)N * 4 + 2 * (size_t)kAsGroups * kAsChunk * 4 + kAsThreads * 8;
}

__global__ __launch_bounds__(kAsThreads) void assign_one_kernel(const AssignArgs p) {
  extern __shared__ __attribute__((aligned(16))) char dsm[];
  const int N = p.N;
  int *s_off = (int *)dsm;                                 // [kAsBlocks][N]
  float *s_q = (float *)(s_off + kAsBlocks * N);           // [N] P partial sums of the blocks before r0
  int *s_part = (int *)(s_q + N);                          // [kAsGroups][kAsChunk]
  float *s_pq = (float *)(s_part + kAsGroups * kAsChunk);  // [kAsGroups][kAsChunk]
  double *s_acc = (double *)(s_pq + kAsGroups * kAsChunk); // [kAsThreads]
  const int tid = threadIdx.x, jq = tid % 32, rg = tid / 32;
  const int64_t Np = count_stride(N);
  const int64_t r0 = (int64_t)blockIdx.x * kAsBlocks, r1 = min(r0 + kAsBlocks, p.nb);
  const bool last = r1 == p.nb;

  // 1. counts (and, for the last group, P partials) of blocks [0, r0)
  for (int c0 = 0; c0 < N; c0 += kAsChunk) {
    const int j4 = c0 + 4 * jq;
    const bool act = j4 < N;  // Np % 4 == 0: the 4 columns from j4 lie inside the row
    int c[4] = {0, 0, 0, 0};
    float q[4] = {0.f, 0.f, 0.f, 0.f};
    if (act) {
      for (int64_t b = rg; b < r0; b += (int64_t)kAsGroups * kAsBatch) {
        u32x4 cv[kAsBatch];
#pragma unroll
        for (int i = 0; i < kAsBatch; ++i)  // clamped past r0: a row that exists, never added
          cv[i] = *(const u32x4 *)(p.bcount + min(b + (int64_t)i * kAsGroups, r0 - 1) * Np + j4);
#pragma unroll
        for (int i = 0; i < kAsBatch; ++i)
          if (b + (int64_t)i * kAsGroups < r0) {
#pragma unroll
            for (int k = 0; k < 4; ++k) c[k] += (int)cv[i][k];
          }
      }
      if (last) {
        for (int64_t b = rg; b < r0; b += (int64_t)kAsGroups * kAsBatch) {
          f32x4 pv[kAsBatch];
#pragma unroll
          for (int i = 0; i < kAsBatch; ++i)
            pv[i] = *(const f32x4 *)(p.ppart + min(b + (int64_t)i * kAsGroups, r0 - 1) * Np + j4);
#pragma unroll
          for (int i = 0; i < kAsBatch; ++i)
            if (b + (int64_t)i * kAsGroups < r0) {
#pragma unroll
              for (int k = 0; k < 4; ++k) q[k] += pv[i][k];
            }
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      s_part[rg * kAsChunk + 4 * jq + k] = c[k];
      s_pq[rg * kAsChunk + 4 * jq + k] = q[k];
    }
    __syncthreads();
    if (tid < kAsChunk && c0 + tid < N) {
      int off = 0;
      float qs = 0.f;
#pragma unroll
      for (int g = 0; g < kAsGroups; ++g) {
        off += s_part[g * kAsChunk + tid];
        qs += s_pq[g * kAsChunk + tid];
      }
      s_off[c0 + tid] = off;
      s_q[c0 + tid] = qs;
    }
    __syncthreads();
  }

  // 2. offsets of each of this group's blocks; the last group's totals
  double acc = 0.0;
  for (int j = tid; j < N; j += kAsThreads) {
    int run = s_off[j];
    float qs = s_q[j];
    for (int64_t b = r0; b < r1; ++b) {
      s_off[(b - r0) * N + j] = run;
      run += p.bcount[b * Np + j];
      if (last) qs += p.ppart[b * Np + j];
    }
    if (last) {
      p.expert_count[j] = run;
      p.psum[j] = qs;
      acc += (double)run * (double)qs;
    }
  }
  if (last) s_acc[tid] = acc;
  __syncthreads();

  // 3. routes: slot = offset of the route's block for its expert + in-block rank
  const int64_t j = r0 * kRouterTokens + tid;
  const int lane = tid % kWave;
  bool drop = false;
  int64_t t, o;
  if (tid < kAsTokens && j < p.nb * kRouterTokens && virt_token(j, p.T, p.Tp, p.k, t, o)) {
    const int e = p.expert_idx[o];
    const int sl = s_off[(tid / kRouterTokens) * N + e] + p.rank[j];
    p.slot[o] = sl;
    drop = sl >= p.C;
    p.dropped[o] = drop ? 1 : 0;
    if (!drop && p.tok) {
      p.tok[(int64_t)e * p.C + sl] = (int32_t)t;
      if (p.rows) p.rows[(int64_t)e * p.C + sl] = (int32_t)o;
      p.gmap[(int64_t)e * p.C + sl] = p.gate[o];
    }
  }
  if (p.y) {
    // one route per token: the output rows of this group's dropped tokens
    // (0, or x with the residual), listed in LDS and written by all threads
    // of the group (16-byte pieces, consecutive threads along a row)
    __shared__ int s_nd;
    int *s_drop = s_part;  // free after step 1
    if (tid == 0) s_nd = 0;
    __syncthreads();
    const unsigned long long mask = __ballot(drop);
    if (mask) {
      int base = 0;
      if (lane == 0) base = atomicAdd(&s_nd, (int)__popcll(mask));
      base = __shfl(base, 0, kWave);
      if (drop) s_drop[base + (int)__popcll(mask & ((1ull << lane) - 1))] = (int)t;
    }
    __syncthreads();
    const int nd = s_nd;
    if (p.gamma) {  // one wave per row
      for (int r = tid / kWave; r < nd; r += kAsThreads / kWave) {
        const int64_t tt = s_drop[r];
        norm_row_wave(p.xres + tt * p.row16, p.y + tt * p.row16, p.row16, p.bf16_, p.gamma, p.beta, p.eps, lane);
      }
    } else {
      for (int it = tid; it < nd * p.row16; it += kAsThreads) {
        const int r = it / p.row16, c = it - r * p.row16;
        const int64_t tt = s_drop[r];
        p.y[tt * p.row16 + c] = p.xres ? p.xres[tt * p.row16 + c] : u32x4{0, 0, 0, 0};
      }
    }
  }

  // 4. loss = N * sum_i (count_i / (k T)) (psum_i / T), reduced in double in a fixed order
  if (last) {
    for (int w = kAsThreads / 2; w > 0; w >>= 1) {
      if (tid < w) s_acc[tid] += s_acc[tid + w];
      __syncthreads();
    }
    if (tid == 0) {
      const double tt = (double)p.T;
      p.aux_loss[0] = (float)(s_acc[0] * (double)N / ((double)p.k * tt * tt));
    }
  }
}

// One launch when the prefix reads of all workgroups together stay small.
// One launch while the prefix rows all workgroups read stay below 64 MB in
// total (base workload: 256 blocks x 128 experts, 16.8 MB).
bool assign_single_launch(int64_t nb, int N) {
  const int64_t groups = ceil_div(nb, kAsBlocks);
  const double reads = 0.5 * (double)groups * (double)(groups * kAsBlocks) * (double)count_stride(N) * 4.0;
  return nb > 0 && reads <= 64.0 * (1 << 20) && assign_one_smem(N) <= 64 * 1024;
}

hipError_t launch_assign(const RouteArgs &a, const LayerMaps &m, hipStream_t st, LaunchMarks marks) {
  auto mark = [&](const char *name) {
    if (marks.fn) marks.fn(marks.ctx, name);
  };
  auto reps = [&]() { return marks.reps ? marks.reps(marks.ctx) : 1; };
  const int64_t nb1 = router_blocks(a.T), nb = a.k * nb1, Tp = nb1 * kRouterTokens;
  hipError_t e;
  if (nb == 0) {
    for (int r = reps(); r > 0; --r)
      route_empty_kernel<<<dim3((unsigned)ceil_div(a.N, 256)), dim3(256), 0, st>>>(a.N, a.expert_count,
                                                                                   a.aux_loss);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    mark("assign");
    return hipSuccess;
  }
  const int row16 = a.d * (a.dtype == kBF16 ? 2 : 4) / 16;
  u32x4 *y = a.k == 1 ? (u32x4 *)m.y : nullptr;
  if (assign_single_launch(nb, a.N)) {
    AssignArgs p{a.expert_idx, a.rank, a.slot, a.dropped, a.bcount, a.ppart, a.T, Tp, nb, a.k, a.N, a.C,
                 a.expert_count, a.psum, a.aux_loss, a.gate, m.tok, m.rows, m.gmap, (const u32x4 *)m.xres, y, row16,
                 a.dtype == kBF16, m.gamma, m.beta, m.eps};
    for (int r = reps(); r > 0; --r)
      assign_one_kernel<<<dim3((unsigned)ceil_div(nb, kAsBlocks)), dim3(kAsThreads), assign_one_smem(a.N), st>>>(p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    mark("assign");
    return hipSuccess;
  }
  for (int r = reps(); r > 0; --r)
    assign_scan_kernel<<<dim3((unsigned)ceil_div(a.N, kWave)), dim3(kScanWaves * kWave), 0, st>>>(
        a.bcount, a.boff, a.ppart, nb, a.N, a.expert_count, a.psum);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  mark("assign_scan");
  const dim3 grid((unsigned)ceil_div(nb * kRouterTokens, 256));
  for (int r = reps(); r > 0; --r) {
    if (m.tok)
      assign_apply_layer_kernel<<<grid, dim3(256), 0, st>>>(
          a.expert_idx, a.rank, a.slot, a.dropped, a.boff, a.T, Tp, a.k, a.N, a.C, a.expert_count, a.psum,
          a.aux_loss, m.tok, m.rows, m.gmap, a.gate,
          DropRows{(const u32x4 *)m.xres, y, row16, a.dtype == kBF16, m.gamma, m.beta, m.eps});
    else
      assign_apply_kernel<<<grid, dim3(256), 0, st>>>(a.expert_idx, a.rank, a.slot, a.dropped, a.boff, a.T, Tp,
                                                      a.k, a.N, a.C, a.expert_count, a.psum, a.aux_loss);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  mark("assign_apply");
  return hipSuccess;
}

}  // namespace smx
