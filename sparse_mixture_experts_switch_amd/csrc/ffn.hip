// Expert FFN of the Switch layer: N independent FFNs, E_i(x) = W_out,i .
// ReLU(W_in,i . x), each run on the rows of its own expert.
//
// Switch Transformers write-up, "The Core Idea: Sparse Activation via
// Routing" (replace the dense FFN by N independent FFNs, only the selected
// expert runs for a token), "Expert Capacity" (fixed per-expert buffers;
// unused slots are padding and carry no work here: expert i has
// M_i = min(count_i, capacity) live rows and the kernels touch no others) and
// the combine equation of "Switch Routing" (y = p_e(x) E_e(x)).
//
// Two grouped GEMMs, both "activations x weights^T" with the contraction
// dimension contiguous in memory for both operands:
//   up:   H_i = ReLU(X_i [M_i x d] . W_in,i^T [d x d_ff])      -> [N][C][d_ff]
//   down: Y_i =      H_i [M_i x d_ff] . W_out,i^T [d_ff x d]
// With ~C rows per expert each weight byte feeds only ~C multiply-adds, so
// both GEMMs are bound by streaming the weights from HBM.  The tiling reads
// every weight byte once: a workgroup owns every live row of one expert (up
// to 16 * MB) and a band of output features; the expert's activation rows
// pass through LDS chunk by chunk while its weight rows stream from global
// memory straight into MFMA operand registers, DEPTH chunks ahead.
//
// Row sources and sinks:
//   A rows come from the [N][C][K] expert buffer, or (gather) from token rows
//   of x through tok[i][r], the token held in slot r of expert i;
//   results go to an [N][C][Nout] buffer (optionally through ReLU), or
//   (combine) straight to y[tok[i][r]] scaled by that token's gate, plus the
//   token's x row when a residual is asked for -- one rounding per output.

#include "common.h"
#include "launch.h"

#include <algorithm>

namespace smx {

constexpr int kFfnThreads = 256;  // fp32 kernel: 4 waves
constexpr int kKC = 64;           // contraction chunk
constexpr int kLdsStride = kKC + 8;

enum Epi { kEpiRelu = 0, kEpiPlain = 1, kEpiCombine = 2 };

template <typename T_>
struct GemmArgs {
  const T_ *A;          // [N][C][K], or x [T][K] when gathering
  const T_ *B;          // [N][Nout][K]
  T_ *Out;              // [N][C][Nout], or y [T][Nout] for the combine epilogue
  const int32_t *counts;
  const int32_t *tok;   // [N][C] token of each live slot (gather / combine)
  const float *gate;    // [T] (combine)
  const T_ *xres;       // [T][Nout] residual rows (combine), or null
  int C, K, Nout, m_tiles, n_tiles, ntiles;
};

// Workgroups are dealt to the 8 XCDs round-robin (workgroup b runs on XCD
// b % 8).  Remap so that each XCD gets a contiguous range of tiles: the tiles
// of one expert then run together on one XCD and share its L2 for the
// expert's activation rows.
__device__ __forceinline__ int xcd_tile(int b, int grid) {
  const int per = grid / 8;  // grid is a multiple of 8
  return (b % 8) * per + b / 8;
}

// bf16 grouped GEMM on v_mfma_f32_16x16x32_bf16.
// MB: 16-row blocks per workgroup; NBW: 16-column blocks per wave;
// WAVES: waves per workgroup (workgroup columns = WAVES * 16 * NBW);
// DEPTH: register ring of contraction chunks in flight.
// Operand layout: lane l supplies row (l % 16) and 8 consecutive k starting
// at 8 * (l / 16); result lane l holds column (l % 16), rows 4 * (l / 16) + i.
template <int MB, int NBW, int DEPTH, int WAVES, bool kGather, int kEpi>
__global__ __launch_bounds__(WAVES * 64) void ffn_gemm_bf16_kernel(const GemmArgs<bf16> p) {
  constexpr int kFfnThreads = WAVES * 64;
  constexpr int kRows = MB * 16;
  constexpr int kCols = WAVES * NBW * 16;
  constexpr int kAChunks = kRows * (kKC / 8);  // 16-byte pieces of one A chunk
  constexpr int kAPer = (kAChunks + kFfnThreads - 1) / kFfnThreads;
  constexpr int kABytes = 2 * kRows * kLdsStride * 2;
  constexpr int kEStride = NBW * 16 + 4;  // fp32 staging row (per wave)
  constexpr int kEBytes = WAVES * 16 * kEStride * 4;
  constexpr int kSmem = kABytes > kEBytes ? kABytes : kEBytes;
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  __shared__ int s_tok[kRows];
  __shared__ float s_gate[kRows];
  bf16 *sA = (bf16 *)smem;

  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  if (tile >= p.ntiles) return;
  const int e = tile / (p.m_tiles * p.n_tiles);
  const int rem = tile % (p.m_tiles * p.n_tiles);
  const int mt = rem / p.n_tiles, nt = rem % p.n_tiles;
  const int M = min(p.counts[e], p.C);
  const int m0 = mt * kRows;
  if (m0 >= M) return;
  const int mrows = min(kRows, M - m0);
  const int amb = (mrows + 15) / 16;
  const int K = p.K, Nout = p.Nout;

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int r16 = lane % 16, kq = (lane / 16) * 8;
  const int ncol0 = nt * kCols + wave * NBW * 16;

  if (kGather || kEpi == kEpiCombine) {
    for (int r = tid; r < mrows; r += kFfnThreads) {
      const int t = p.tok[(int64_t)e * p.C + m0 + r];
      s_tok[r] = t;
      if (kEpi == kEpiCombine) s_gate[r] = p.gate[t];
    }
    __syncthreads();
  }

  // Weight rows of this wave (rows past Nout read row 0; never stored).
  const bf16 *bp[NBW];
  bool bval[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const int n = ncol0 + nb * 16 + r16;
    bval[nb] = n < Nout;
    bp[nb] = p.B + ((int64_t)e * Nout + (bval[nb] ? n : 0)) * K + kq;
  }
  // Activation pieces this thread moves into LDS: row ar[q], 8 columns at
  // ac[q].  Rows past the live ones re-read the last live row, so that every
  // lane always loads (no divergent branches around the loads: the compiler
  // can then count outstanding loads exactly and keep the prefetch in flight).
  const bf16 *asrc[kAPer];
  int aoff[kAPer];
#pragma unroll
  for (int q = 0; q < kAPer; ++q) {
    const int i = (tid + q * kFfnThreads) % kAChunks;
    const int r = i / (kKC / 8), c = i % (kKC / 8);
    const int rr = min(r, mrows - 1);
    asrc[q] = (kGather ? p.A + (int64_t)s_tok[rr] * K : p.A + ((int64_t)e * p.C + m0 + rr) * K) + c * 8;
    aoff[q] = r * kLdsStride + c * 8;
  }

  f32x4 acc[MB][NBW];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nch = K / kKC;
  u32x4 areg[DEPTH][kAPer];
  u32x4 breg[DEPTH][2][NBW];
  // Loads of chunk `ch` (clamped to the last chunk past the end: re-reads
  // that hit in cache and are never consumed).
  auto fetch = [&](int slot, int ch) {
    const int k0 = min(ch, nch - 1) * kKC;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) breg[slot][s][nb] = *(const u32x4 *)(bp[nb] + k0 + s * 32);
#pragma unroll
    for (int q = 0; q < kAPer; ++q) areg[slot][q] = *(const u32x4 *)(asrc[q] + k0);
  };
  auto store_a = [&](int slot, int buf) {
#pragma unroll
    for (int q = 0; q < kAPer; ++q) *(u32x4 *)(&sA[buf * kRows * kLdsStride + aoff[q]]) = areg[slot][q];
  };

#pragma unroll
  for (int j = 0; j < DEPTH; ++j) fetch(j, j);
  store_a(0, 0);
  __syncthreads();
  for (int base = 0; base < nch; base += DEPTH) {
#pragma clang loop unroll(full)
    for (int j = 0; j < DEPTH; ++j) {
      const int ch = base + j;
      if (ch < nch) {
        const bf16 *abuf = sA + (ch & 1) * kRows * kLdsStride;
#pragma clang loop unroll(full)
        for (int s = 0; s < 2; ++s) {
          // every row block runs: rows past the live ones hold copies of the
          // last live row and are never stored (straight-line MFMA stream;
          // the kernel is bound by the weight stream, not by MFMA)
#pragma clang loop unroll(full)
          for (int mb = 0; mb < MB; ++mb) {
            const bf16x8 a = as_bf16x8(*(const u32x4 *)(&abuf[(mb * 16 + r16) * kLdsStride + s * 32 + kq]));
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb)
              acc[mb][nb] =
                  __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(breg[j][s][nb]), acc[mb][nb], 0, 0, 0);
          }
        }
      }
      // refill this ring slot DEPTH chunks ahead, then move the next chunk's
      // activations into the other LDS buffer (its readers finished at the
      // previous barrier)
      fetch(j, ch + DEPTH);
      store_a((j + 1) % DEPTH, (ch + 1) & 1);
      __syncthreads();
    }
  }

  // Epilogue: per 16-row block, each wave stages its 16 x (16 NBW) fp32 tile
  // in LDS, then writes whole 16-byte row pieces.
  float *stg = (float *)smem + wave * 16 * kEStride;
  constexpr int kPieces = NBW * 2;  // 8-column pieces per staged row
  // fully unrolled so that acc is only ever indexed by constants
#pragma clang loop unroll(full)
  for (int mb = 0; mb < MB; ++mb) {
    if (mb >= amb) continue;
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) stg[((lane / 16) * 4 + i) * kEStride + nb * 16 + r16] = acc[mb][nb][i];
    __syncthreads();
    for (int c = lane; c < 16 * kPieces; c += kWave) {
      const int rr = c / kPieces, pc = c % kPieces;
      const int m = mb * 16 + rr;
      const int n = ncol0 + pc * 8;
      if (m < mrows && n < Nout) {
        const f32x4 v0 = *(const f32x4 *)&stg[rr * kEStride + pc * 8];
        const f32x4 v1 = *(const f32x4 *)&stg[rr * kEStride + pc * 8 + 4];
        float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        bf16x8 o;
        if (kEpi == kEpiCombine) {
          const int t = s_tok[m];
          const float g = s_gate[m];
          bf16x8 xv{};
          if (p.xres) xv = as_bf16x8(*(const u32x4 *)(p.xres + (int64_t)t * Nout + n));
#pragma unroll
          for (int i = 0; i < 8; ++i) o[i] = (bf16)(p.xres ? (float)xv[i] + g * v[i] : g * v[i]);
          *(u32x4 *)(p.Out + (int64_t)t * Nout + n) = as_u32x4(o);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) o[i] = (bf16)(kEpi == kEpiRelu ? fmaxf(v[i], 0.f) : v[i]);
          *(u32x4 *)(p.Out + ((int64_t)e * p.C + m0 + m) * Nout + n) = as_u32x4(o);
        }
      }
    }
    __syncthreads();
  }
}

// fp32 grouped GEMM on the vector ALUs: 64 x 64 output tiles, 16-deep
// contraction slices staged in LDS, 4 x 4 outputs per thread.
template <bool kGather, int kEpi>
__global__ __launch_bounds__(kFfnThreads) void ffn_gemm_f32_kernel(const GemmArgs<float> p) {
  constexpr int kT = 64, kKs = 16;
  __shared__ float sA[kKs][kT + 1], sB[kKs][kT + 1];
  __shared__ int s_tok[kT];
  __shared__ float s_gate[kT];
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  if (tile >= p.ntiles) return;
  const int e = tile / (p.m_tiles * p.n_tiles);
  const int rem = tile % (p.m_tiles * p.n_tiles);
  const int mt = rem / p.n_tiles, nt = rem % p.n_tiles;
  const int M = min(p.counts[e], p.C);
  const int m0 = mt * kT, n0 = nt * kT;
  if (m0 >= M) return;
  const int K = p.K, Nout = p.Nout;
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  if (kGather || kEpi == kEpiCombine) {
    for (int r = tid; r < kT; r += kFfnThreads)
      if (m0 + r < M) {
        const int t = p.tok[(int64_t)e * p.C + m0 + r];
        s_tok[r] = t;
        if (kEpi == kEpiCombine) s_gate[r] = p.gate[t];
      }
    __syncthreads();
  }
  const float *Aexp = p.A + (int64_t)e * p.C * K;
  const float *Bexp = p.B + (int64_t)e * Nout * K;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += kKs) {
    for (int i = tid; i < kT * kKs; i += kFfnThreads) {
      const int r = i / kKs, k = i % kKs;
      const int m = m0 + r, n = n0 + r;
      float av = 0.f;
      if (m < M) av = kGather ? p.A[(int64_t)s_tok[r] * K + k0 + k] : Aexp[(int64_t)m * K + k0 + k];
      sA[k][r] = av;
      sB[k][r] = (n < Nout) ? Bexp[(int64_t)n * K + k0 + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kKs; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = sA[k][ty * 4 + i];
        b[i] = sB[k][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ty * 4 + i, m = m0 + r;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= Nout) continue;
      const float v = acc[i][j];
      if (kEpi == kEpiCombine) {
        const int t = s_tok[r];
        const float g = s_gate[r];
        p.Out[(int64_t)t * Nout + n] = p.xres ? p.xres[(int64_t)t * Nout + n] + g * v : g * v;
      } else {
        p.Out[((int64_t)e * p.C + m) * Nout + n] = kEpi == kEpiRelu ? fmaxf(v, 0.f) : v;
      }
    }
  }
}

namespace {

constexpr int kMaxMB = 10;  // up to 160 live rows per workgroup

int pick_mb(int C) {
  const int need = (int)ceil_div(std::min(C, kMaxMB * 16), 16);
  static const int opts[] = {1, 2, 4, 6, 8, 10};
  for (int o : opts)
    if (o >= need) return o;
  return kMaxMB;
}

template <typename T_>
GemmArgs<T_> make_args(const GemmCall &c, int rows, int cols) {
  GemmArgs<T_> g;
  g.A = (const T_ *)c.A;
  g.B = (const T_ *)c.B;
  g.Out = (T_ *)c.Out;
  g.counts = c.counts;
  g.tok = c.tok;
  g.gate = c.gate;
  g.xres = (const T_ *)c.xres;
  g.C = c.C;
  g.K = c.K;
  g.Nout = c.Nout;
  g.m_tiles = (int)ceil_div(c.C, rows);
  g.n_tiles = (int)ceil_div(c.Nout, cols);
  g.ntiles = c.N * g.m_tiles * g.n_tiles;
  return g;
}

inline unsigned grid_of(int ntiles) { return (unsigned)(ceil_div(ntiles, 8) * 8); }

// Tile shape (measured on MI355X for the weight-streaming regime): every
// live row of the expert (up to 160) x 384 output features per workgroup of
// 8 waves (3 column blocks each), two contraction chunks in flight.
constexpr int kNBW = 3, kWaves = 8, kDepth = 2;

template <int MB, bool kGather, int kEpi>
hipError_t run_bf16(const GemmCall &c, hipStream_t st) {
  auto g = make_args<bf16>(c, MB * 16, kWaves * 16 * kNBW);
  ffn_gemm_bf16_kernel<MB, kNBW, kDepth, kWaves, kGather, kEpi>
      <<<dim3(grid_of(g.ntiles)), dim3(kWaves * 64), 0, st>>>(g);
  return hipGetLastError();
}

template <bool kGather, int kEpi>
hipError_t gemm(const GemmCall &c, hipStream_t st) {
  if (c.N == 0 || c.C == 0) return hipSuccess;
  if (c.dtype == kF32) {
    auto g = make_args<float>(c, 64, 64);
    ffn_gemm_f32_kernel<kGather, kEpi><<<dim3(grid_of(g.ntiles)), dim3(kFfnThreads), 0, st>>>(g);
    return hipGetLastError();
  }
  switch (pick_mb(c.C)) {
    case 1: return run_bf16<1, kGather, kEpi>(c, st);
    case 2: return run_bf16<2, kGather, kEpi>(c, st);
    case 4: return run_bf16<4, kGather, kEpi>(c, st);
    case 6: return run_bf16<6, kGather, kEpi>(c, st);
    case 8: return run_bf16<8, kGather, kEpi>(c, st);
    default: return run_bf16<10, kGather, kEpi>(c, st);
  }
}

}  // namespace

// Stage call: dispatched buffer -> H -> expert_out buffer.
hipError_t launch_ffn_up(const FfnArgs &a, hipStream_t st) {
  GemmCall c{a.dtype, a.N, a.C, a.d, a.dff, a.dispatched, a.w_in, a.hidden, a.expert_count,
             nullptr, nullptr, nullptr};
  return gemm<false, kEpiRelu>(c, st);
}

hipError_t launch_ffn_down(const FfnArgs &a, hipStream_t st) {
  GemmCall c{a.dtype, a.N, a.C, a.dff, a.d, a.hidden, a.w_out, a.expert_out, a.expert_count,
             nullptr, nullptr, nullptr};
  return gemm<false, kEpiPlain>(c, st);
}

// Layer path: token rows of x gathered through tok -> H; H -> y scattered
// through tok with the gate (and residual) applied.
hipError_t launch_ffn_up_gather(const GemmCall &c, hipStream_t st) { return gemm<true, kEpiRelu>(c, st); }
hipError_t launch_ffn_down_combine(const GemmCall &c, hipStream_t st) { return gemm<false, kEpiCombine>(c, st); }

}  // namespace smx
