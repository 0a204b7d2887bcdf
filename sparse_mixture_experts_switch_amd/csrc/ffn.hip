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
// memory straight into MFMA operand registers, two chunks ahead.  The
// weights are either row-major or tiled (stored in MFMA operand order, see
// tile.hip); both give the same operands in the same lanes.
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
#include <atomic>

namespace smx {

int device_cus() {
  static std::atomic<int> cache[kMaxDeviceCache];
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  const bool cached = dev >= 0 && dev < kMaxDeviceCache;
  if (cached && (cus = cache[dev].load(std::memory_order_relaxed)) > 0) return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
  if (cached) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

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
  const float *gate;    // [T] (combine, fp32 path)
  const float *gmap;    // [N][C] gate of the token in each live slot (combine, bf16 path)
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

// bf16 grouped GEMM on v_mfma_f32_16x16x32_bf16, persistent.
//
// A workgroup stays resident and walks a list of tiles (one expert's live
// rows [m0, m0 + mrows) x kCols output features).  XCD x (= blockIdx % 8,
// workgroups are dealt to the 8 XCDs round-robin) owns a contiguous range of
// tiles, so the tiles of one expert run together on one XCD and share its L2
// for the expert's activation rows; empty tiles are skipped.
//
// The contraction runs in 64-column chunks.  Weight rows stream from global
// memory straight into MFMA operand registers through a two-chunk register
// ring; activation rows pass through a double-buffered padded LDS tile.  The
// ring runs on across tile boundaries: the next tile's first chunks are in
// flight while the current tile finishes and while its results are written,
// so a tile change costs no pipeline refill.
//
// MB: 16-row blocks per tile; NBW: 16-column blocks per wave; WAVES: waves
// per workgroup (kCols = WAVES * 16 * NBW).  Operand layout: lane l supplies
// row (l % 16) and 8 consecutive k starting at 8 * (l / 16); result lane l
// holds column (l % 16), rows 4 * (l / 16) + i.
//
// kTiled: the weights are stored in that operand order (16-row x 32-column
// blocks, each 64 lanes x 16 bytes), so a wave's weight load of one block
// is one contiguous 1 KB piece; row-major weights make every load touch 16
// rows, which costs the vector memory path several times the cycles.
// kStream (one row tile per expert, so every weight byte is read once):
// tiled weights are loaded nontemporally, leaving the 256 MB last-level
// cache to the hidden activations and token rows that the other product
// re-reads (measured on both products together; either alone gains
// nothing).  kNtOut: the results are stored nontemporally, written back as
// they go instead of left dirty in L2, whose evictions would then mix
// write-backs into the weight stream (H, and y when it outgrows the L2s);
// results that fit the L2s are better stored normally and written back in
// one piece when the kernel ends.  With several row tiles per expert the
// tiles re-read the expert's weights and the down-projection re-reads H
// from cache: ordinary loads and stores.
template <int MB, int NBW, int WAVES, bool kGather, int kEpi, bool kTiled, bool kStream, bool kNtOut,
          bool kSkipDead = true>
__global__ __launch_bounds__(WAVES * 64) void ffn_gemm_bf16_kernel(const GemmArgs<bf16> p) {
  constexpr int kThreads = WAVES * 64;
  constexpr int kRows = MB * 16;
  constexpr int kCols = WAVES * NBW * 16;
  constexpr int kAChunks = kRows * (kKC / 8);  // 16-byte pieces of one A chunk
  constexpr int kAPer = (kAChunks + kThreads - 1) / kThreads;
  constexpr int kAStage = kRows * kLdsStride;  // bf16 per LDS buffer
  constexpr int kEStride = NBW * 16 + 4;       // fp32 staging row (per wave)
  constexpr int kPieces = NBW * 2;             // 8-column pieces per staged row
  // Output rows of the expert buffer (not the combine): 16-row blocks of the
  // whole tile are staged (double-buffered) and written in whole rows
  constexpr bool kWholeRows = kEpi != kEpiCombine;
  constexpr int kWStride = kCols + 16;         // fp32 staging row of the whole tile
  constexpr int kRowPieces = kCols / 8;        // 8-column pieces per tile row
  constexpr int kStageFloats = kWholeRows ? 2 * 16 * kWStride : WAVES * 16 * kEStride;
  constexpr bool kTok = kGather || kEpi == kEpiCombine;
  static_assert(kRows <= kThreads, "one row per thread for the tile's token map");
  __shared__ __attribute__((aligned(16))) bf16 sA[2 * kAStage];
  __shared__ __attribute__((aligned(16))) float sStage[kStageFloats];
  __shared__ int s_tok[2][kRows];
  __shared__ float s_gate[2][kRows];

  const int K = p.K, Nout = p.Nout, C = p.C;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int r16 = lane % 16, kq = (lane / 16) * 8;
  const int nch = K / kKC;
  const int nchp = nch + (nch & 1);  // chunks per tile, padded to the ring depth

  // ---- tile schedule (uniform) ----
  const int g8 = gridDim.x / 8, xcd = blockIdx.x % 8, lid = blockIdx.x / 8;
  const int per = (p.ntiles + 7) / 8;
  const int t_end = min(p.ntiles, (xcd + 1) * per);
  int t_next = xcd * per + lid;
  struct Tile {
    int e, m0, n0, mrows;
  };
  auto next_tile = [&](Tile &t) -> bool {
    while (t_next < t_end) {
      const int id = t_next;
      t_next += g8;
      const int e = id / (p.m_tiles * p.n_tiles);
      const int rem = id % (p.m_tiles * p.n_tiles);
      const int m0 = (rem / p.n_tiles) * kRows;
      const int M = min(p.counts[e], C);
      if (m0 < M) {
        t.e = e;
        t.m0 = m0;
        t.n0 = (rem % p.n_tiles) * kCols;
        t.mrows = min(kRows, M - m0);
        return true;
      }
    }
    return false;
  };

  // ---- per-lane pieces of the activation chunk: row ar[q], columns ac[q] ----
  int ar[kAPer], aoff[kAPer];
#pragma unroll
  for (int q = 0; q < kAPer; ++q) {
    const int i = (tid + q * kThreads) % kAChunks;
    ar[q] = i / (kKC / 8);
    aoff[q] = ar[q] * kLdsStride + (i % (kKC / 8)) * 8;
  }
  // Token of each of this lane's activation rows, for the current and the
  // next tile (gather); rows past the live ones re-read the last live row so
  // that every lane always loads (branch-free loads keep the ring counted).
  int atok[2][kAPer];
  auto load_atok = [&](int which, const Tile &t) {
#pragma unroll
    for (int q = 0; q < kAPer; ++q) atok[which][q] = p.tok[(int64_t)t.e * C + t.m0 + min(ar[q], t.mrows - 1)];
  };
  // Token and gate of row `tid` of a tile (combine epilogue).
  int ttok = 0;
  float tgate = 0.f;
  auto load_rowinfo = [&](const Tile &t) {
    const int64_t sl = (int64_t)t.e * C + t.m0 + min(tid, t.mrows - 1);
    ttok = p.tok[sl];
    if (kEpi == kEpiCombine) tgate = p.gmap[sl];
  };

  Tile cur, nxt;
  if (!next_tile(cur)) return;
  bool have_nxt = next_tile(nxt);

  u32x4 areg[2][kAPer];
  u32x4 breg[2][2][NBW];
  // Loads of chunk `ch` of tile t (clamped to the tile's last chunk past its
  // end: re-reads that hit in cache and are never consumed).  Activation rows
  // are issued first: loads complete in issue order, and the activations are
  // needed one iteration before the weights.
  auto fetch = [&](int slot, const Tile &t, int which, int ch) {
    const int k0 = min(ch, nch - 1) * kKC;
#pragma unroll
    for (int q = 0; q < kAPer; ++q) {
      const int64_t row = kGather ? (int64_t)atok[which][q] : (int64_t)t.e * C + t.m0 + min(ar[q], t.mrows - 1);
      areg[slot][q] = *(const u32x4 *)(p.A + row * K + (aoff[q] % kLdsStride) + k0);
    }
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      if (kTiled) {
        const int blk = min((t.n0 + wave * NBW * 16 + nb * 16) / 16, Nout / 16 - 1);
        const bf16 *bp = p.B + (((int64_t)t.e * (Nout / 16) + blk) * (K / 32) + k0 / 32) * 512 + lane * 8;
#pragma unroll
        for (int s = 0; s < 2; ++s)
          breg[slot][s][nb] = kStream ? __builtin_nontemporal_load((const u32x4 *)(bp + s * 512))
                                      : *(const u32x4 *)(bp + s * 512);
      } else {
        const int n = min(t.n0 + wave * NBW * 16 + nb * 16 + r16, Nout - 1);
        const bf16 *bp = p.B + ((int64_t)t.e * Nout + n) * K + kq + k0;
#pragma unroll
        for (int s = 0; s < 2; ++s) breg[slot][s][nb] = *(const u32x4 *)(bp + s * 32);
      }
    }
  };
  auto store_a = [&](int slot, int buf) {
#pragma unroll
    for (int q = 0; q < kAPer; ++q) *(u32x4 *)(&sA[buf * kAStage + aoff[q]]) = areg[slot][q];
  };

  // ---- prologue: token maps of the first two tiles, first two chunks ----
  int cb = 0;  // s_tok / s_gate buffer of the current tile
  if (kGather) {
    load_atok(0, cur);
    if (have_nxt) load_atok(1, nxt);
  }
  if (kTok) {
    load_rowinfo(cur);
    if (tid < kRows) {  // rows past mrows hold a valid copy of the last live row
      s_tok[0][tid] = ttok;
      if (kEpi == kEpiCombine) s_gate[0][tid] = tgate;
    }
    if (have_nxt) load_rowinfo(nxt);
  }
  fetch(0, cur, 0, 0);
  fetch(1, cur, 0, 1);
  store_a(0, 0);
  __syncthreads();

  while (true) {
    // ---- one tile: `cur` ----
    const int mlive = (cur.mrows + 15) / 16;  // row blocks holding live rows (uniform)
    f32x4 acc[MB][NBW];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int base = 0; base < nchp; base += 2) {
#pragma clang loop unroll(full)
      for (int j = 0; j < 2; ++j) {
        const int ch = base + j;
        if (ch < nch) {
          const bf16 *abuf = sA + j * kAStage;
#pragma clang loop unroll(full)
          for (int s = 0; s < 2; ++s) {
            auto blocks = [&](int mb0, int mb1) {
#pragma clang loop unroll(full)
              for (int mb = mb0; mb < mb1; ++mb) {
                const bf16x8 a = as_bf16x8(*(const u32x4 *)(&abuf[(mb * 16 + r16) * kLdsStride + s * 32 + kq]));
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb)
                  acc[mb][nb] =
                      __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(breg[j][s][nb]), acc[mb][nb], 0, 0, 0);
              }
            };
            // Row blocks past the live ones hold copies of the last live row
            // and are never stored.  The last two pairs of blocks run only
            // when they hold live rows (two uniform branches; finer-grained
            // skipping breaks up the MFMA stream and costs more than it saves).
            if (kSkipDead && MB >= 6) {
              blocks(0, MB - 4);
              if (mlive > MB - 4) blocks(MB - 4, MB - 2);
              if (mlive > MB - 2) blocks(MB - 2, MB);
            } else {
              blocks(0, MB);
            }
          }
        }
        // refill this ring slot two chunks ahead (the next tile's first
        // chunks once this tile's run out), then move the next chunk's
        // activations into the other LDS buffer
        if (ch + 2 < nchp || !have_nxt)
          fetch(j, cur, 0, ch + 2);
        else
          fetch(j, nxt, 1, ch + 2 - nchp);
        store_a(j ^ 1, j ^ 1);
        __syncthreads();
      }
    }

    // ---- epilogue of `cur` ----
    auto put = [&](bf16 *dst, const bf16x8 &o) {
      if (kNtOut)
        __builtin_nontemporal_store(as_u32x4(o), (u32x4 *)dst);
      else
        *(u32x4 *)dst = as_u32x4(o);
    };
    if (kWholeRows) {
      // Rows of the [N][C][Nout] buffer: each 16-row block of the tile is
      // staged for the whole workgroup, and consecutive threads write
      // consecutive 16-byte pieces of whole tile rows, so every wave stores
      // whole cache lines (per-wave pieces of 96 bytes leave lines to be
      // written back in parts: 135 MB written for 101 MB of H).  Two staging
      // buffers, one LDS-only barrier per block: a wave overwrites a buffer
      // only after the next block's barrier, which every wave reaches after
      // its reads of it.  Measured at 16384 tokens, d_model 768, d_ff 3072,
      // 128 experts: the up-projection 140.7 -> 132.6 us.
      int sb = 0;
#pragma clang loop unroll(full)
      for (int mb = 0; mb < MB; ++mb) {
        if (mb >= mlive) continue;
        float *stg = sStage + sb * 16 * kWStride;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            stg[((lane / 16) * 4 + i) * kWStride + wave * NBW * 16 + nb * 16 + r16] = acc[mb][nb][i];
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // LDS only: stores keep going
        for (int c = tid; c < 16 * kRowPieces; c += kThreads) {
          const int rr = c / kRowPieces, pc = c % kRowPieces;
          const int m = mb * 16 + rr;
          const int n = cur.n0 + pc * 8;
          if (m < cur.mrows && n < Nout) {
            const f32x4 v0 = *(const f32x4 *)&stg[rr * kWStride + pc * 8];
            const f32x4 v1 = *(const f32x4 *)&stg[rr * kWStride + pc * 8 + 4];
            const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            bf16x8 o;
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = (bf16)(kEpi == kEpiRelu ? fmaxf(v[i], 0.f) : v[i]);
            put(p.Out + ((int64_t)cur.e * C + cur.m0 + m) * Nout + n, o);
          }
        }
        sb ^= 1;
      }
      // the next tile's epilogue reuses the buffers after its chunk barriers
    } else {
      // The combine: rows go to scattered tokens of y; each wave stages
      // 16-row blocks of its columns in its own LDS region and writes whole
      // 16-byte row pieces (staging the whole tile as above measured no
      // faster here)
      float *stg = sStage + wave * 16 * kEStride;
      const int ncol0 = cur.n0 + wave * NBW * 16;
#pragma clang loop unroll(full)
      for (int mb = 0; mb < MB; ++mb) {
        if (mb >= mlive) continue;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) stg[((lane / 16) * 4 + i) * kEStride + nb * 16 + r16] = acc[mb][nb][i];
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's staging writes landed
        __builtin_amdgcn_wave_barrier();
        for (int c = lane; c < 16 * kPieces; c += kWave) {
          const int rr = c / kPieces, pc = c % kPieces;
          const int m = mb * 16 + rr;
          const int n = ncol0 + pc * 8;
          if (m < cur.mrows && n < Nout) {
            const f32x4 v0 = *(const f32x4 *)&stg[rr * kEStride + pc * 8];
            const f32x4 v1 = *(const f32x4 *)&stg[rr * kEStride + pc * 8 + 4];
            const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            const int t = s_tok[cb][m];
            const float g = s_gate[cb][m];
            bf16x8 xv{}, o;
            if (p.xres) xv = as_bf16x8(*(const u32x4 *)(p.xres + (int64_t)t * Nout + n));
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = (bf16)(p.xres ? (float)xv[i] + g * v[i] : g * v[i]);
            put(p.Out + (int64_t)t * Nout + n, o);
          }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // staging reads done before the next block overwrites
        __builtin_amdgcn_wave_barrier();
      }
    }

    if (!have_nxt) break;
    // ---- advance: nxt becomes cur; look up the tile after it ----
    cur = nxt;
    cb ^= 1;
    if (kTok) {
      // rowinfo of the new cur was loaded a whole tile ago; publish it (the
      // next barrier, inside the first chunk, makes it visible)
      if (tid < kRows) {
        s_tok[cb][tid] = ttok;
        if (kEpi == kEpiCombine) s_gate[cb][tid] = tgate;
      }
    }
    if (kGather) {
#pragma unroll
      for (int q = 0; q < kAPer; ++q) atok[0][q] = atok[1][q];
    }
    have_nxt = next_tile(nxt);
    if (have_nxt) {
      if (kGather) load_atok(1, nxt);
      if (kTok) load_rowinfo(nxt);
    }
  }
}

// fp32 grouped GEMM on the vector ALUs: 64 x 64 output tiles, 32-deep
// contraction slices staged in LDS, 4 x 4 outputs per thread.  The next
// three slices are in registers while the current one is multiplied, so a
// tile pays about one global-load round trip per three slices, not one per
// slice (small fp32 layers have few tiles, and each tile's slices run in
// sequence).
template <bool kGather, int kEpi>
__global__ __launch_bounds__(kFfnThreads) void ffn_gemm_f32_kernel(const GemmArgs<float> p) {
  constexpr int kT = 64, kKs = 32;
  constexpr int kLd = kT * kKs / kFfnThreads;  // elements of each operand per thread and slice
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
  // slices s, s + 1, s + 2 in flight in a register ring (slot s mod 3; the
  // loop is unrolled by the ring depth so that every slot index is a
  // constant): small layers have short contractions, and one slice of
  // products does not cover a global-load round trip
  constexpr int kRing = 3;
  float ra[kRing][kLd], rb[kRing][kLd];
  auto load = [&](int slot, int k0) {  // K is a multiple of 64: every slice is whole
#pragma unroll
    for (int q = 0; q < kLd; ++q) {
      const int i = tid + q * kFfnThreads;
      const int r = i / kKs, k = i % kKs;
      const int m = m0 + r, n = n0 + r;
      ra[slot][q] = m < M ? (kGather ? p.A[(int64_t)s_tok[r] * K + k0 + k] : Aexp[(int64_t)m * K + k0 + k]) : 0.f;
      rb[slot][q] = n < Nout ? Bexp[(int64_t)n * K + k0 + k] : 0.f;
    }
  };
  float acc[4][4] = {};
  const int ns = K / kKs;
#pragma unroll
  for (int j = 0; j < kRing; ++j)
    if (j < ns) load(j, j * kKs);
  for (int s0 = 0; s0 < ns; s0 += kRing) {
#pragma unroll
    for (int j = 0; j < kRing; ++j) {
      const int sl = s0 + j;
      if (sl < ns) {
        __syncthreads();  // the previous slice's products are done with the LDS tiles
#pragma unroll
        for (int q = 0; q < kLd; ++q) {
          const int i = tid + q * kFfnThreads;
          sA[i % kKs][i / kKs] = ra[j][q];
          sB[i % kKs][i / kKs] = rb[j][q];
        }
        __syncthreads();
        if (sl + kRing < ns) load(j, (sl + kRing) * kKs);
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
            for (int jj = 0; jj < 4; ++jj) acc[i][jj] = __builtin_fmaf(a[i], b[jj], acc[i][jj]);
        }
      }
    }
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
  g.gmap = c.gmap;
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
// 8 waves (3 column blocks each), or x 256 features (2 column blocks) when
// that spreads the output features more evenly over the CUs.
constexpr int kWaves = 8;

// Resident workgroups for a persistent launch: CUs x workgroups per CU.  The
// occupancy is queried once per device and kernel: occ_cache belongs to the
// calling instantiation (all the kernels share one function type, so a
// static here would be shared by every tile shape).
template <typename Kern>
unsigned persistent_grid(Kern kern, int ntiles, std::atomic<int> (&occ_cache)[kMaxDeviceCache]) {
  const int cus = device_cus();
  int dev = 0, occ = 0;
  const bool cached = hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDeviceCache;
  if (cached) occ = occ_cache[dev].load(std::memory_order_relaxed);
  if (occ < 1) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, kWaves * 64, 0) != hipSuccess || occ < 1) occ = 1;
    if (cached) occ_cache[dev].store(occ, std::memory_order_relaxed);
  }
  const int64_t want = std::min<int64_t>((int64_t)cus * occ, ceil_div(ntiles, 8) * 8);
  return (unsigned)std::max<int64_t>(8, ceil_div(want, 8) * 8);
}

template <int MB, int NBW, bool kGather, int kEpi, bool kTiled, bool kStream, bool kNtOut>
hipError_t run_bf16(const GemmCall &c, hipStream_t st) {
  static std::atomic<int> occ[kMaxDeviceCache];
  auto g = make_args<bf16>(c, MB * 16, kWaves * 16 * NBW);
  auto kern = ffn_gemm_bf16_kernel<MB, NBW, kWaves, kGather, kEpi, kTiled, kStream, kNtOut>;
  kern<<<dim3(persistent_grid(kern, g.ntiles, occ)), dim3(kWaves * 64), 0, st>>>(g);
  return hipGetLastError();
}

// Rows of y that the combine stores normally when streaming: y of at most
// 28 MiB fits the eight XCDs' 4 MiB L2s with room to spare.  Measured with
// tiled weights, back to back / cold: 16384 tokens x d_model 768 (24 MiB of
// y) 277 -> 273 / 283 -> 277.5 us with ordinary stores; 16384 x 1024 (32
// MiB) 307 -> 310 / 311 -> 314 us and 8192 x 4096 (64 MiB) 2050 -> 2081 /
// 2044 -> 2078 us, so nontemporal there.
constexpr int64_t kKeepOutBytes = int64_t(28) << 20;

template <int MB, int NBW, bool kGather, int kEpi, bool kTiled>
hipError_t run_bf16_stream(const GemmCall &c, hipStream_t st) {
  if constexpr (kEpi == kEpiCombine) {
    if (c.out_rows * c.Nout * 2 <= kKeepOutBytes) return run_bf16<MB, NBW, kGather, kEpi, kTiled, true, false>(c, st);
  }
  return run_bf16<MB, NBW, kGather, kEpi, kTiled, true, true>(c, st);
}

// Row tiles per expert: one unless the capacity exceeds the largest tile
// (MB = kMaxMB); only then are the weights re-read (measured at 16384 tokens,
// d_model 768, d_ff 3072, 128 experts, tiled weights: streaming takes the
// layer from 316 to 290 us at capacity 160, and would take the top-2 layer
// at capacity 320 from 504 to 577 us).
template <int MB, int NBW, bool kGather, int kEpi>
hipError_t run_bf16(const GemmCall &c, hipStream_t st) {
  bool stream = true;
  if constexpr (MB == kMaxMB) stream = ceil_div(c.C, MB * 16) == 1;
  if (c.tiled)
    return stream ? run_bf16_stream<MB, NBW, kGather, kEpi, true>(c, st)
                  : run_bf16<MB, NBW, kGather, kEpi, true, false, false>(c, st);
  return stream ? run_bf16_stream<MB, NBW, kGather, kEpi, false>(c, st)
                : run_bf16<MB, NBW, kGather, kEpi, false, false, false>(c, st);
}

// Column blocks per wave.  Both widths stream every weight byte once and run
// at the same speed per output feature (measured); what differs is how many
// feature columns the busiest CU gets when the tiles are dealt out (e.g. 1024
// features: 3 tiles of 384 per expert leave half the CUs with two tiles,
// 4 tiles of 256 give every CU the same).  Ties keep the wider tile, which
// re-reads each expert's activation rows fewer times.
int pick_nbw(const GemmCall &c, int rows) {
  const int cus = device_cus();
  auto span = [&](int nbw) {
    const int64_t cols = (int64_t)kWaves * 16 * nbw;
    const int64_t tiles = (int64_t)c.N * ceil_div(c.C, rows) * ceil_div(c.Nout, cols);
    return ceil_div(tiles, cus) * cols;
  };
  return span(2) < span(3) ? 2 : 3;
}

template <int MB, bool kGather, int kEpi>
hipError_t run_bf16_mb(const GemmCall &c, hipStream_t st) {
  return pick_nbw(c, MB * 16) == 2 ? run_bf16<MB, 2, kGather, kEpi>(c, st) : run_bf16<MB, 3, kGather, kEpi>(c, st);
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
    case 1: return run_bf16_mb<1, kGather, kEpi>(c, st);
    case 2: return run_bf16_mb<2, kGather, kEpi>(c, st);
    case 4: return run_bf16_mb<4, kGather, kEpi>(c, st);
    case 6: return run_bf16_mb<6, kGather, kEpi>(c, st);
    case 8: return run_bf16_mb<8, kGather, kEpi>(c, st);
    default: return run_bf16_mb<10, kGather, kEpi>(c, st);
  }
}

}  // namespace

// Stage call: dispatched buffer -> H -> expert_out buffer.
hipError_t launch_ffn_up(const FfnArgs &a, hipStream_t st) {
  GemmCall c{a.dtype, a.N, a.C, a.d, a.dff, a.dispatched, a.w_in, a.hidden, a.expert_count,
             nullptr, nullptr, nullptr, nullptr, a.tiled};
  return gemm<false, kEpiRelu>(c, st);
}

hipError_t launch_ffn_down(const FfnArgs &a, hipStream_t st) {
  GemmCall c{a.dtype, a.N, a.C, a.dff, a.d, a.hidden, a.w_out, a.expert_out, a.expert_count,
             nullptr, nullptr, nullptr, nullptr, a.tiled};
  return gemm<false, kEpiPlain>(c, st);
}

// Layer path: token rows of x gathered through tok -> H; H -> y scattered
// through tok with the gate (and residual) applied.
hipError_t launch_ffn_up_gather(const GemmCall &c, hipStream_t st) { return gemm<true, kEpiRelu>(c, st); }
hipError_t launch_ffn_down_combine(const GemmCall &c, hipStream_t st) { return gemm<false, kEpiCombine>(c, st); }

}  // namespace smx
