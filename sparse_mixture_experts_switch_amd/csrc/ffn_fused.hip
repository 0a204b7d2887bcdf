// Expert FFN and combine in one pass: y[t] = g_t W_out,e ReLU(W_in,e x_t)
// (+ x_t) for the kept tokens of every expert, without writing the hidden
// activations to memory.
//
// Switch Transformers write-up, "The Core Idea: Sparse Activation via
// Routing" (the dense FFN replaced by N independent FFNs E_i(x) =
// W_out,i ReLU(W_in,i x)), "Expert Capacity" (each expert runs on the tokens
// in its buffer: the M_i = min(count_i, capacity) kept ones) and the combine
// equation of "Switch Routing" (y = p_e(x) E_e(x), k = 1).
//
// A workgroup owns a tile of up to 80 kept rows of one expert and every one
// of the d_model output features of those rows (d_model 128 or 256); an
// expert with more than 80 kept rows has two tiles, placed on the same XCD so
// that the second reader of each weight byte finds it in that XCD's L2.  The
// tile walks d_ff in chunks of 128:
//   up:   H_c = ReLU(X W_in[c]^T)      [rows x 128], computed transposed
//         (W_in rows are the MFMA row operand, token rows the column
//         operand), so that each lane's four results are four consecutive
//         d_ff values of one token and go to LDS as one 8-byte store in the
//         operand order of the next product; wave w computes d_ff columns
//         [32 w, 32 w + 32) of the chunk, so each X operand read from LDS
//         feeds two MFMAs;
//   down: Y += H_c W_out[:, c]^T       [rows x d_model], accumulated in
//         registers: wave w owns d_model columns [16 NB w, 16 NB (w + 1)).
// Four waves, one per SIMD, each with the SIMD's whole register file: the
// MFMA results stay in the accumulation registers, and the kernel pipelines
// explicitly instead of relying on a second wave per SIMD: operands for the
// next step are read from LDS before the current step's MFMAs, and weight
// operands stream from memory straight into registers through a ring of RING
// loads per wave that runs across the two products and across chunks (each
// load's place in the instruction stream is pinned).
//
// Where it pays (measured, 16384 tokens, 128 experts, capacity 160, bf16):
// d_model 128 / d_ff 512: 35 us against 46 us for the up- and down-projection
// kernels; 256 / 1024: 64 against 68 us; 512 / 2048: 192 against 191 us;
// 768 / 3072: 389 against 332 us.  Each workgroup streams the whole of its
// expert's two weight matrices (both tiles of an expert read them, once from
// memory and once from L2), twice the bytes per CU of the two-kernel layout,
// so at large d_model the bytes it can keep in flight per CU (the operand
// ring lives in registers beside the output tile) set its speed; the layer
// call takes it for d_model 128 and 256 only.
// The tile's token rows X (gathered from x through the slot -> token map)
// stay in LDS for the whole tile, laid out in MFMA operand order (each
// operand read is 1 KB of consecutive bytes).  H never leaves the chip:
// against an up-projection that writes H and a down-projection that reads it
// back, this saves 2 x kept x d_ff x 2 bytes of traffic and, more, the write
// stream that slows the weight reads it is mixed with.
//
// MFMA v_mfma_f32_16x16x32_bf16: operand lane l supplies row (l % 16) and the
// 8 contraction values from 8 * (l / 16); result lane l holds column
// (l % 16), rows 4 * (l / 16) + i.

#include "common.h"
#include "launch.h"

namespace smx {

constexpr int kFzChunk = 128;            // d_ff columns per chunk
constexpr int kFzMaxMB = 5;              // 16-row blocks per tile (80 rows)

struct FusedArgs {
  const bf16 *x;        // [T][d]
  const bf16 *w_in;     // [N][f][d]
  const bf16 *w_out;    // [N][d][f]
  bf16 *out;            // output rows [.][d]
  const int32_t *counts;
  const int32_t *tok;   // [N][C] token of each live slot
  const int32_t *rows;  // [N][C] output row of each live slot, or null (= tok)
  const float *gmap;    // [N][C] gate of each live slot
  const bf16 *xres;     // residual rows [T][d] (added to row tok), or null
  const float *gamma, *beta;  // Add + Normalize epilogue (with xres = x)
  float eps;
  int C, f, m_tiles, ntiles;
  bool tiled;           // w_in / w_out in MFMA operand order (16 x 32 blocks of 64 lanes x 16 bytes)
};

// LDS-only barrier: waits for this wave's LDS operations, not for its
// outstanding global loads (a __syncthreads would also drain the weight ring).
__device__ __forceinline__ void fz_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Keeps the instructions before it ahead of those after it (the scheduler
// would otherwise sink the ring's refills to the end of a product).
__device__ __forceinline__ void fz_pin() { __builtin_amdgcn_sched_barrier(0); }

// Each of the four waves computes CB = 2 column blocks of 16 of the chunk's H.
constexpr int kFzWaves = 4;

template <int MB, int NB, int RING, bool kNorm, bool kTiled>
__global__ __launch_bounds__(kFzWaves * 64) void ffn_fused_bf16_kernel(const FusedArgs p) {
  constexpr int CB = kFzChunk / 16 / kFzWaves;
  constexpr int D = NB * 16 * kFzWaves;     // d_model
  constexpr int KS = D / 32;                // contraction steps of the up-projection
  constexpr int DS = kFzChunk / 32;         // contraction steps of the down-projection per chunk
  constexpr int LU = CB * KS;               // up-projection loads per chunk
  constexpr int L = LU + DS * NB;           // weight operand loads per chunk per wave
  constexpr int kFzThreads = kFzWaves * 64;
  static_assert(L % RING == 0, "ring positions must repeat every chunk");
  constexpr int kRows = MB * 16;
  constexpr int kXBytes = MB * KS * 1024;   // X in operand order
  constexpr int kHBytes = MB * DS * 1024;   // one chunk of H in operand order
  constexpr int kEStride = NB * 16 + 4;     // epilogue staging row (fp32), per wave
  constexpr int kStgBytes = kFzWaves * 16 * kEStride * 4;
  constexpr int kNormBytes = 16 * (D + 4) * 4;
  constexpr int kEpiBytes = kStgBytes > kNormBytes ? kStgBytes : kNormBytes;
  constexpr int kXRegion = kXBytes > kEpiBytes ? kXBytes : kEpiBytes;  // X, then the epilogue staging
  __shared__ __attribute__((aligned(16))) char smem[kXRegion + kHBytes];
  char *sx = smem;
  char *sh = smem + kXRegion;
  // the accumulators live in the MFMA accumulation registers
  asm volatile("" ::: "a0");

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int r16 = lane % 16, kq = (lane / 16) * 8;

  // ---- tile: XCD x (= blockIdx % 8) owns a contiguous range of tiles, so
  // the tiles of one expert share an L2 ----
  const int per = gridDim.x / 8;
  const int tile = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (tile >= p.ntiles) return;
  const int e = tile / p.m_tiles;
  const int m0 = (tile % p.m_tiles) * kRows;
  const int M = min(p.counts[e], p.C);
  if (m0 >= M) return;
  const int mrows = min(kRows, M - m0);
  const int f = p.f, nch = f / kFzChunk;
  const int64_t slot0 = (int64_t)e * p.C + m0;

  // ---- weight operand streams of this wave ----
  // up, load (s, cb) of chunk c: W_in row e*f + c*128 + 16*(CB*wave + cb) + r16,
  //   columns 32 s + kq
  // down, load (ks, nb) of chunk c: W_out row e*D + wave*NB*16 + nb*16 + r16,
  //   columns c*128 + 32 ks + kq
  // (tiled weights: the same operands as whole 1 KB blocks, block
  // (row / 16, column / 32) of the expert's matrix)
  const bf16 *win = kTiled ? p.w_in + ((int64_t)e * (f / 16) + CB * wave) * (D / 32) * 512 + lane * 8
                           : p.w_in + ((int64_t)e * f + 16 * CB * wave + r16) * D + kq;
  const bf16 *wout = kTiled ? p.w_out + ((int64_t)e * (D / 16) + wave * NB) * (f / 32) * 512 + lane * 8
                            : p.w_out + ((int64_t)e * D + wave * NB * 16 + r16) * f + kq;
  u32x4 ring[RING];
  auto load = [&](int i, int c) {  // load i (compile-time after unrolling) of chunk c
    const int cc = min(c, nch - 1);  // past the last chunk: re-read it (never consumed)
    if (i < LU) {
      const int s = i / CB, cb = i % CB;
      ring[i % RING] = kTiled ? *(const u32x4 *)(win + ((int64_t)(cc * (kFzChunk / 16) + cb) * (D / 32) + s) * 512)
                              : *(const u32x4 *)(win + ((int64_t)cc * kFzChunk + 16 * cb) * D + 32 * s);
    } else {
      const int u = i - LU, ks = u / NB, nb = u % NB;
      ring[i % RING] = kTiled ? *(const u32x4 *)(wout + ((int64_t)nb * (f / 32) + cc * (kFzChunk / 32) + ks) * 512)
                              : *(const u32x4 *)(wout + (int64_t)nb * 16 * f + cc * kFzChunk + 32 * ks);
    }
  };
  // issue the load RING places ahead of load i of chunk c
  auto refill = [&](int i, int c) { load(i + RING < L ? i + RING : i + RING - L, i + RING < L ? c : c + 1); };

  // ---- stage X: piece q -> operand (mb, s), lane ll: token row mb*16 + ll%16,
  // columns 32 s + 8 (ll / 16) ----
  {
    constexpr int kPieces = MB * KS * 64;
    constexpr int kPer = (kPieces + kFzThreads - 1) / kFzThreads;
    // the first RING weight loads go out first: they take longest
#pragma unroll
    for (int i = 0; i < RING; ++i) load(i, 0);
#pragma unroll
    for (int q0 = 0; q0 < kPer; q0 += 8) {  // 8 pieces per thread in flight at a time
      u32x4 xv[8];
#pragma unroll
      for (int q = q0; q < q0 + 8 && q < kPer; ++q) {
        const int i = min(tid + q * kFzThreads, kPieces - 1);
        const int ll = i % 64, fs = i / 64, mb = fs / KS, s = fs % KS;
        const int r = min(mb * 16 + ll % 16, mrows - 1);  // rows past the live ones copy the last live row
        const int t = p.tok[slot0 + r];
        xv[q - q0] = *(const u32x4 *)(p.x + (int64_t)t * D + 32 * s + 8 * (ll / 16));
      }
#pragma unroll
      for (int q = q0; q < q0 + 8 && q < kPer; ++q) {
        const int i = tid + q * kFzThreads;
        if (i < kPieces) *(u32x4 *)(sx + (int64_t)i * 16) = xv[q - q0];
      }
    }
  }
  fz_barrier();

  f32x4 yacc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) yacc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // H store position of this lane for its column block cb: the block's d_ff
  // columns start at q = 16 (CB wave + cb) in the chunk, so operand (mb,
  // ks = q / 32), lane r16 + 16 (2 ((q % 32) / 16) + (lane / 16) / 2), byte
  // 8 ((lane / 16) % 2)
  auto hpos = [&](int cb) {
    const int q = 16 * (CB * wave + cb);
    return (q / 32) * 1024 + (r16 + 16 * (2 * ((q % 32) / 16) + lane / 32)) * 16 + 8 * ((lane / 16) % 2);
  };
  auto xfrag = [&](int mb, int s) { return as_bf16x8(*(const u32x4 *)(sx + ((mb * KS + s) * 64 + lane) * 16)); };
  auto hfrag = [&](int mb, int ks) { return as_bf16x8(*(const u32x4 *)(sh + ((mb * DS + ks) * 64 + lane) * 16)); };

  for (int c = 0; c < nch; ++c) {
    // ---- up: H_c^T = W_in[c] X^T, CB column blocks ----
    f32x4 uacc[MB][CB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) uacc[mb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 xb[2][MB];  // this step's operands and the next step's, read ahead
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) xb[0][mb] = xfrag(mb, 0);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      bf16x8 a[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        a[cb] = as_bf16x8(ring[(CB * s + cb) % RING]);
        refill(CB * s + cb, c);
      }
      if (s + 1 < KS) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) xb[(s + 1) & 1][mb] = xfrag(mb, s + 1);
      }
      fz_pin();
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          uacc[mb][cb] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[cb], xb[s & 1][mb], uacc[mb][cb], 0, 0, 0);
      fz_pin();
    }
    // ReLU, bf16, into LDS in the down-projection's operand order
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 h;
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = (bf16)fmaxf(uacc[mb][cb][i], 0.f);
        *(bf16x4 *)(sh + mb * DS * 1024 + hpos(cb)) = h;
      }
    fz_barrier();  // H_c complete
    // ---- down: Y += H_c W_out[:, c]^T ----
    bf16x8 hb[2][MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) hb[0][mb] = hfrag(mb, 0);
#pragma unroll
    for (int ks = 0; ks < DS; ++ks) {
      if (ks + 1 < DS) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) hb[(ks + 1) & 1][mb] = hfrag(mb, ks + 1);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int i = LU + ks * NB + nb;
        const bf16x8 b = as_bf16x8(ring[i % RING]);
        refill(i, c);
        fz_pin();
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          yacc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hb[ks & 1][mb], b, yacc[mb][nb], 0, 0, 0);
        fz_pin();
      }
    }
    fz_barrier();  // H_c consumed
  }

  const int mlive = (mrows + 15) / 16;
  if constexpr (kNorm) {
    // ---- epilogue with the block's Add + Normalize ("The Architecture in
    // Place"): out row = (v - mean) / sqrt(var + eps) * gamma + beta with
    // v = x + g * acc over all D features.  Each 16-row block is staged in
    // fp32 by all waves in the (now free) X region; then each wave takes four
    // rows: per-lane partial sums in piece order and fixed-order butterflies
    // for the mean and the squared deviations, one rounding per output ----
    constexpr int kRowF = D + 4;     // staged row pitch (floats)
    constexpr int kP = (D / 8 + kWave - 1) / kWave;  // 8-value pieces per lane
    float *srow = (float *)sx;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (mb >= mlive) continue;  // uniform
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          srow[((lane / 16) * 4 + i) * kRowF + wave * NB * 16 + nb * 16 + r16] = yacc[mb][nb][i];
      fz_barrier();
      for (int rr = wave; rr < 16; rr += kFzWaves) {
        const int m = mb * 16 + rr;
        if (m >= mrows) continue;  // uniform per wave
        const int t = p.tok[slot0 + m];
        const float g = p.gmap[slot0 + m];
        float v[kP][8];
        float sum = 0.f;
#pragma unroll
        for (int q = 0; q < kP; ++q) {
          const int cpc = lane + q * kWave;
          if (cpc < D / 8) {
            const bf16x8 xv = as_bf16x8(*(const u32x4 *)(p.xres + (int64_t)t * D + cpc * 8));
            const f32x4 a0 = *(const f32x4 *)&srow[rr * kRowF + cpc * 8];
            const f32x4 a1 = *(const f32x4 *)&srow[rr * kRowF + cpc * 8 + 4];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              v[q][k] = (float)xv[k] + g * (k < 4 ? a0[k] : a1[k - 4]);
              sum += v[q][k];
            }
          }
        }
        const float mean = wave_sum(sum) / (float)D;
        float sq = 0.f;
#pragma unroll
        for (int q = 0; q < kP; ++q)
          if (lane + q * kWave < D / 8) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              const float dv = v[q][k] - mean;
              sq += dv * dv;
            }
          }
        const float rstd = 1.0f / sqrtf(wave_sum(sq) / (float)D + p.eps);
#pragma unroll
        for (int q = 0; q < kP; ++q) {
          const int cpc = lane + q * kWave;
          if (cpc < D / 8) {
            bf16x8 o;
#pragma unroll
            for (int k = 0; k < 8; ++k)
              o[k] = (bf16)((v[q][k] - mean) * rstd * p.gamma[cpc * 8 + k] + p.beta[cpc * 8 + k]);
            *(u32x4 *)(p.out + (int64_t)t * D + cpc * 8) = as_u32x4(o);
          }
        }
      }
      fz_barrier();  // staged rows read before the next block overwrites them
    }
    return;
  }

  // ---- epilogue: y row = g * acc (+ x row); each wave stages 16-row blocks
  // of its columns in its own part of the (now free) X region and writes
  // whole 16-byte row pieces ----
  constexpr int kPc = NB * 2;  // 8-column pieces per staged row
  float *stg = (float *)sx + wave * 16 * kEStride;
  const int ncol0 = wave * NB * 16;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    if (mb >= mlive) continue;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) stg[((lane / 16) * 4 + i) * kEStride + nb * 16 + r16] = yacc[mb][nb][i];
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's staging writes landed
    __builtin_amdgcn_wave_barrier();
    for (int q = lane; q < 16 * kPc; q += kWave) {
      const int rr = q / kPc, pc = q % kPc;
      const int m = mb * 16 + rr;
      if (m < mrows) {
        const int n = ncol0 + pc * 8;
        const int t = p.tok[slot0 + m];
        const int64_t orow = p.rows ? p.rows[slot0 + m] : t;
        const float g = p.gmap[slot0 + m];
        const f32x4 v0 = *(const f32x4 *)&stg[rr * kEStride + pc * 8];
        const f32x4 v1 = *(const f32x4 *)&stg[rr * kEStride + pc * 8 + 4];
        const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        bf16x8 o;
        if (p.xres) {
          const bf16x8 xv = as_bf16x8(*(const u32x4 *)(p.xres + (int64_t)t * D + n));
#pragma unroll
          for (int i = 0; i < 8; ++i) o[i] = (bf16)((float)xv[i] + g * v[i]);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) o[i] = (bf16)(g * v[i]);
        }
        *(u32x4 *)(p.out + orow * D + n) = as_u32x4(o);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // staging reads done before the next block overwrites
    __builtin_amdgcn_wave_barrier();
  }
}

namespace {

template <int MB, int D>
hipError_t run_fused(const FusedArgs &a, hipStream_t st) {
  constexpr int NB = D / 16 / kFzWaves;                  // output column blocks per wave
  constexpr int L = 2 * (D / 32) + 4 * NB;                // weight loads per chunk per wave
  constexpr int RING = L % 32 == 0 ? 32 : (L % 16 == 0 ? 16 : 8);
  const unsigned grid = (unsigned)(ceil_div(a.ntiles, 8) * 8);
  auto kern = a.gamma ? (a.tiled ? ffn_fused_bf16_kernel<MB, NB, RING, true, true>
                                 : ffn_fused_bf16_kernel<MB, NB, RING, true, false>)
                      : (a.tiled ? ffn_fused_bf16_kernel<MB, NB, RING, false, true>
                                 : ffn_fused_bf16_kernel<MB, NB, RING, false, false>);
  kern<<<dim3(grid), dim3(kFzWaves * 64), 0, st>>>(a);
  return hipGetLastError();
}

template <int D>
hipError_t run_fused_mb(const FusedArgs &a, int mb, hipStream_t st) {
  switch (mb) {
    case 1: return run_fused<1, D>(a, st);
    case 2: return run_fused<2, D>(a, st);
    case 3: return run_fused<3, D>(a, st);
    case 4: return run_fused<4, D>(a, st);
    default: return run_fused<5, D>(a, st);
  }
}

}  // namespace

bool ffn_fused_eligible(int dtype, int d, int dff, int C) {
  return dtype == kBF16 && (d == 128 || d == 256) && dff % kFzChunk == 0 && dff > 0 && C > 0 &&
         C <= 2 * kFzMaxMB * 16;
}

hipError_t launch_ffn_fused(const FusedFfnCall &c, hipStream_t st) {
  if (c.N == 0 || c.C == 0) return hipSuccess;
  if (!ffn_fused_eligible(c.dtype, c.d, c.dff, c.C)) return hipErrorInvalidValue;
  // rows per tile: all of an expert's capacity in one tile when it fits,
  // else two tiles of equal 16-row blocks
  const int blocks = (int)ceil_div(c.C, 16);
  const int mb = blocks <= kFzMaxMB ? blocks : (int)ceil_div(blocks, 2);
  if (c.gamma && (c.rows || !c.xres)) return hipErrorInvalidValue;  // normalization: one route per token, x given
  FusedArgs a{(const bf16 *)c.x, (const bf16 *)c.w_in, (const bf16 *)c.w_out, (bf16 *)c.out, c.counts, c.tok,
              c.rows, c.gmap, (const bf16 *)c.xres, c.gamma, c.beta, c.eps, c.C, c.dff,
              (int)ceil_div(c.C, mb * 16), 0, c.tiled};
  a.ntiles = c.N * a.m_tiles;
  return c.d == 128 ? run_fused_mb<128>(a, mb, st) : run_fused_mb<256>(a, mb, st);
}

}  // namespace smx
