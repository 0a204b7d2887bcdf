// Backward pass of the Switch layer: the grouped GEMMs of the experts.
//
// Switch Transformers write-up, "Switch Routing: From Top-k to k = 1": the
// gate p_e(x) multiplies the chosen expert's output, which keeps the router
// differentiable; "Making Sparse Training Stable" (selective precision: the
// router's arithmetic stays in fp32, the experts run in bf16).  With L the
// caller's loss and dy = dL/dy, for a kept token t of expert e with gate g,
// u = W_in,e x, h = ReLU(u) (the forward's saved H) and z = W_out,e^T dy:
//   dL/dg = <z, h>               (= <dy, W_out,e h>)
//   du    = g z * [h > 0]        (dL/du)
//   dW_out,e += (g dy) h^T,  dW_in,e += du x^T,  dx_t += W_in,e^T du.
// Per expert, with the expert's kept rows stacked in slot order:
//   DZ: Z = DY W_out,e           rows x d_ff, contraction d     (B k-major)
//   DX: DX_e = DU W_in,e         rows x d,    contraction d_ff  (B k-major)
//   DWO: dW_out,e = (G DY)^T H   d x d_ff,    contraction rows  (A, B k-major)
//   DWI: dW_in,e = DU^T X        d_ff x d,    contraction rows  (A, B k-major)
// "k-major" operands are stored with the contraction index as the row; the
// MFMA wants 8 consecutive contraction values per lane, so those tiles are
// staged in LDS as stored (16-byte row pieces) and read with the gfx950 LDS
// transpose load (ds_read_b64_tr_b16): within each group of 16 lanes, lane
// 4r + q reads 4 consecutive elements of LDS row r at column 4q, and lane j
// receives element j % 4 of the reads of lanes j / 4, 4 + j / 4, 8 + j / 4,
// 12 + j / 4 -- that is, column j of the 4-row block, rows 0..3.  Two such
// loads give a lane its 8 contraction values.
//
// One workgroup computes one (expert, row tile, column tile); both operands
// pass through LDS (double-buffered with a two-deep register prefetch for the
// long contractions, single-buffered with several workgroups per CU for the
// weight gradients).  Rows of an expert past its kept count are never stored;
// contraction rows past it (DWO / DWI) are zero, so an expert with no kept
// token gets exact zero gradients.  The router's matrix products of the
// backward (W_r^T dL/dh and dW_r) are here too, on exact bf16 plane splits of
// their fp32 operands.  Results are deterministic: fixed tiles, fixed
// reduction order.

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace smx {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

namespace {

constexpr int kBKC = 64;           // contraction columns per chunk
constexpr int kKcStride = kBKC + 8;  // LDS row of a k-contiguous tile (bf16)

// Two transposed LDS loads -> the 8 contraction values of one MFMA operand.
__device__ __forceinline__ bf16x8 tr_operand(const bf16 *tile, int stride, int k0, int c0, int lane) {
  const int g = lane / 16, i = lane % 16;
  const bf16 *p = tile + (k0 + 8 * g + i / 4) * stride + c0 + 4 * (i % 4);
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p + 4 * stride));
  const u32x4 v{__builtin_bit_cast(u32x2v, lo)[0], __builtin_bit_cast(u32x2v, lo)[1],
                __builtin_bit_cast(u32x2v, hi)[0], __builtin_bit_cast(u32x2v, hi)[1]};
  return as_bf16x8(v);
}

}  // namespace

// Operand tile loader.  A tile covers R rows (output rows for A, output
// columns for B) and kBKC contraction columns.
//  KM = false (k-contiguous): element (r, k) at base + row(r) * ld + k; LDS
//    [R][kKcStride]; rows past the live count re-read the last live row.
//  KM = true (k-major): element (r, k) at base + krow(k) * ld + r; LDS
//    [kBKC][R + 8]; contraction rows past the live count are stored as zero.
// With G, rows (KC) or contraction rows (KM) go through the slot -> token
// map, read from an LDS copy (`rows`, indexed from the tile's first row or
// the segment's first contraction row), so that a fetch issues its global
// loads without waiting for any; S scales k-major rows by the slot's gate
// (LDS copy `gates`) when they are stored.  NT makes the loads nontemporal:
// an expert weight matrix is streamed once per kernel, and keeping it out of
// the last-level cache leaves H and DU (100 MB each at the base workload,
// read again by the weight-gradient kernels) there.  fetch() only issues
// loads: every use of the loaded data (zeroing, scaling) happens in store(),
// so loads of later chunks stay in flight.
template <int R, int kThreads, bool KM, bool G, bool S, bool NT = false>
struct TileLoader {
  static constexpr int kPieces = R * kBKC / 8;
  static constexpr int kPer = (kPieces + kThreads - 1) / kThreads;
  static constexpr int kStride = KM ? R + 8 : kKcStride;
  static constexpr int kElems = KM ? kBKC * kStride : R * kStride;
  using Regs = u32x4[kPer];
  int off[kPer];  // LDS element offset of each piece
  int rk[kPer];   // row (KC) or contraction row within the chunk (KM)
  int col[kPer];  // column element offset within the row piece
  bool act[kPer];

  __device__ __forceinline__ void plan(int tid) {
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int i = tid + q * kThreads;
      act[q] = i < kPieces;
      const int ii = act[q] ? i : 0;  // idle pieces load a duplicate of piece 0 and store nothing
      if (KM) {
        rk[q] = ii / (R / 8);
        col[q] = (ii % (R / 8)) * 8;
      } else {
        rk[q] = ii / (kBKC / 8);
        col[q] = (ii % (kBKC / 8)) * 8;
      }
      off[q] = rk[q] * kStride + col[q];
    }
  }

  // KC: rows r0 + rk (live count `live`), contraction chunk at k0.
  // KM: contraction rows k0 + rk (live count `live`, segment start ks),
  //     columns c0 + col (clamped below rmax).
  __device__ __forceinline__ void fetch(Regs &reg, const bf16 *base, int ld, const int *rows, int r0, int c0,
                                        int live, int k0, int ks, int rmax) const {
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      if (KM) {
        const int kk = min(k0 + rk[q], live - 1);
        const int64_t row = G ? (int64_t)rows[kk - ks] : kk;
        const int c = min(c0 + col[q], rmax - 8);
        const u32x4 *src = (const u32x4 *)(base + row * ld + c);
        reg[q] = NT ? __builtin_nontemporal_load(src) : *src;
      } else {
        const int r = min(r0 + rk[q], live - 1);
        const int64_t row = G ? (int64_t)rows[r - r0] : r;
        reg[q] = *(const u32x4 *)(base + row * ld + k0 + col[q]);
      }
    }
  }

  __device__ __forceinline__ void store(const Regs &reg, bf16 *lds, int k0, int live, int ks,
                                        const float *gates) const {
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      if (!act[q]) continue;
      u32x4 v = reg[q];
      if (KM) {
        const int k = k0 + rk[q];
        if (S) {
          const float g = gates[min(k, live - 1) - ks];
          bf16x8 b = as_bf16x8(v);
#pragma unroll
          for (int j = 0; j < 8; ++j) b[j] = (bf16)(g * (float)b[j]);
          v = as_u32x4(b);
        }
        if (k >= live) v = u32x4{0, 0, 0, 0};
      }
      *(u32x4 *)(lds + off[q]) = v;
    }
  }
};

// Epilogues: DU (du = g z [H > 0] and the partial dots <z, H>), DX (the
// experts' part of dx, fp32 rows through the slot -> token map), DW (a weight
// gradient tile), DXR (the router's part of dx plus the experts' part for kept
// tokens plus dy with the residual, rounded once: the whole dx).
enum BwdEpi { kEpiDU = 0, kEpiDX = 1, kEpiDW = 2, kEpiDXR = 3 };

template <typename T_>
struct BwdArgs {
  int C;
  const int32_t *counts;  // [N] routed tokens per expert (kept = min(count, C))
  const int32_t *tok;     // [N][C] token of each live slot
  const float *gmap;      // [N][C] gate of each live slot
  const T_ *A;
  int64_t a_estride;      // elements per expert (non-gathered operands)
  int lda;
  const T_ *B;
  int64_t b_estride;
  int ldb;
  int M, Nout, K;         // fixed dimensions (the live row count replaces M for DU / DX, K for DW)
  void *Out;
  int64_t o_estride;
  int ldo;
  const T_ *H;            // [N][C][Nout] forward hidden activations (DU)
  float *dgpart;          // [T][n_tiles] partial <z, h> per token (DU)
  const float *dxe;       // [T][Nout] experts' part of dx (DXR)
  const uint8_t *dropped; // [T] (DXR)
  const T_ *dyres;        // [T][Nout] dy when the residual is added, or null (DXR)
  int m_tiles, n_tiles;
  int64_t ntiles;
};

// MBW x NBW MFMA blocks per wave, WM x WN waves.  kBufs LDS operand buffers
// and kPre register sets: (2, 2) keeps two contraction chunks in flight while
// the MFMAs consume a third (long contractions); (1, 1) stages one chunk at a
// time and leaves LDS for a second workgroup per CU (short contractions, whose
// workgroups overlap each other instead).  kWavesPerEU (0: none) caps the
// registers so that many waves fit.
template <int MBW, int NBW, int WM, int WN, bool AKM, bool AG, bool AS, bool BKM, bool BG, int EPI, int kBufs,
          int kPre, int kWavesPerEU>
__global__ __launch_bounds__(WM *WN * 64) __attribute__((amdgpu_waves_per_eu(kWavesPerEU > 0 ? kWavesPerEU : 1)))
void bwd_gemm_bf16_kernel(const BwdArgs<bf16> p) {
  constexpr int kThreads = WM * WN * 64;
  constexpr int BM = WM * MBW * 16, BN = WN * NBW * 16;
  constexpr bool kRaggedM = EPI == kEpiDU || EPI == kEpiDX;  // rows = an expert's kept slots
  constexpr bool kRaggedK = EPI == kEpiDW;                   // contraction = an expert's kept slots
  static_assert((kBufs == 2 && (kPre == 1 || kPre == 2)) || (kBufs == 1 && kPre == 1), "pipeline shape");
  using LA = TileLoader<BM, kThreads, AKM, AG, AS>;
  // B is the expert weight matrix in DZ (W_out) and DX (W_in)
  using LB = TileLoader<BN, kThreads, BKM, BG, false, EPI == kEpiDU || EPI == kEpiDX>;
  constexpr int kStageStride = NBW * 16 + 4;  // fp32 epilogue staging row (per wave)
  constexpr int kOperandElems = kBufs * (LA::kElems + LB::kElems);
  constexpr int kStageElems = WM * WN * 16 * kStageStride * 2;  // in bf16 units
  constexpr int kSmem = kOperandElems > kStageElems ? kOperandElems : kStageElems;
  __shared__ __attribute__((aligned(16))) bf16 smem[kSmem];
  __shared__ float s_dg[WN][BM];

  // XCD-aware tile order: blocks b, b + 8, ... run on one XCD; XCD x takes
  // the contiguous tile range [x per, (x + 1) per) so that the tiles of an
  // expert share one L2.
  const int64_t per = (p.ntiles + 7) / 8;
  const int64_t id = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (id >= p.ntiles || blockIdx.x / 8 >= per) return;
  const int e = (int)(id / ((int64_t)p.m_tiles * p.n_tiles));
  const int rem = (int)(id % ((int64_t)p.m_tiles * p.n_tiles));
  const int mt = rem / p.n_tiles, nt = rem % p.n_tiles;
  const int live = (kRaggedM || kRaggedK) ? min(p.counts[e], p.C) : 0;
  const int m0 = mt * BM, n0 = nt * BN;
  const int Mt = kRaggedM ? live : p.M;
  if (m0 >= Mt) return;  // dead tile (ragged rows)
  const int Kt = kRaggedK ? live : p.K;
  const int64_t eC = (int64_t)e * p.C;

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wm = wave / WN, wn = wave % WN;
  const int r16 = lane % 16, kq = (lane / 16) * 8;

  LA la;
  LB lb;
  la.plan(tid);
  lb.plan(tid);
  auto sA = [&](int b) { return smem + b * LA::kElems; };
  auto sB = [&](int b) { return smem + kBufs * LA::kElems + b * LB::kElems; };
  const bf16 *Ab = p.A + (AG ? 0 : (int64_t)e * p.a_estride);
  const bf16 *Bb = p.B + (BG ? 0 : (int64_t)e * p.b_estride);

  // slot -> token copies in LDS: the tile's rows (k-contiguous gathered
  // operands) and one segment of contraction rows with their gates (k-major
  // gathered operands)
  constexpr bool kRowG = (AG && !AKM) || (BG && !BKM);
  constexpr bool kKG = (AG && AKM) || (BG && BKM);
  constexpr int kSeg = 1024;  // contraction rows per segment
  __shared__ int s_rtok[kRowG ? (BM > BN ? BM : BN) : 1];
  __shared__ int s_ktok[kKG ? kSeg : 1];
  __shared__ float s_kgate[(kKG && AS) ? kSeg : 1];
  if (kRowG) {
    const int r0 = (AG && !AKM) ? m0 : n0, lv = (AG && !AKM) ? Mt : p.Nout;
    for (int r = tid; r < ((AG && !AKM) ? BM : BN); r += kThreads) s_rtok[r] = p.tok[eC + min(r0 + r, lv - 1)];
    __syncthreads();
  }

  typename LA::Regs ra[kPre];
  typename LB::Regs rb[kPre];
  int ks = 0;  // first contraction row of the current segment
  // A rows: output rows (KC: live count Mt) or output rows with contraction
  // rows live up to Kt (KM).  B likewise with the output columns.
  auto fetch = [&](auto slot, int k0) {
    constexpr int sl = decltype(slot)::value;
    if (AKM)
      la.fetch(ra[sl], Ab, p.lda, s_ktok, 0, m0, Kt, k0, ks, p.M);
    else
      la.fetch(ra[sl], Ab, p.lda, s_rtok, m0, 0, Mt, k0, ks, 0);
    if (BKM)
      lb.fetch(rb[sl], Bb, p.ldb, s_ktok, 0, n0, Kt, k0, ks, p.Nout);
    else
      lb.fetch(rb[sl], Bb, p.ldb, s_rtok, n0, 0, p.Nout, k0, ks, 0);
  };
  int kst = 0;  // contraction row of the chunk being stored
  auto store = [&](auto slot, int buf) {
    constexpr int sl = decltype(slot)::value;
    la.store(ra[sl], sA(buf), kst, Kt, ks, s_kgate);
    lb.store(rb[sl], sB(buf), kst, Kt, ks, s_kgate);
  };

  f32x4 acc[MBW][NBW];
#pragma unroll
  for (int i = 0; i < MBW; ++i)
#pragma unroll
    for (int j = 0; j < NBW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 a[MBW], b[NBW];
#pragma unroll
      for (int i = 0; i < MBW; ++i) {
        const int r = wm * MBW * 16 + i * 16;
        if (AKM)
          a[i] = tr_operand(sA(buf), LA::kStride, s * 32, r, lane);
        else
          a[i] = as_bf16x8(*(const u32x4 *)(sA(buf) + (r + r16) * LA::kStride + s * 32 + kq));
      }
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        const int c = wn * NBW * 16 + j * 16;
        if (BKM)
          b[j] = tr_operand(sB(buf), LB::kStride, s * 32, c, lane);
        else
          b[j] = as_bf16x8(*(const u32x4 *)(sB(buf) + (c + r16) * LB::kStride + s * 32 + kq));
      }
#pragma unroll
      for (int i = 0; i < MBW; ++i)
#pragma unroll
        for (int j = 0; j < NBW; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  // contraction segments: one for fixed contractions; k-major gathered
  // operands take kSeg rows at a time (their token copy is per segment)
  for (ks = 0; ks < Kt; ks += kSeg) {
    const int kend = kKG ? min(Kt, ks + kSeg) : Kt;
    if (kKG) {
      __syncthreads();  // the previous segment's readers are done
      for (int i = tid; i < kend - ks; i += kThreads) {
        s_ktok[i] = p.tok[eC + ks + i];
        if (AS) s_kgate[i] = p.gmap[eC + ks + i];
      }
      __syncthreads();
    }
    const int nch = (int)ceil_div(kend - ks, kBKC);
    if constexpr (kBufs == 2) {
      fetch(I0{}, ks);
      kst = ks;
      store(I0{}, 0);
      if (kPre == 2 && nch > 1) fetch(I1{}, ks + kBKC);
      __syncthreads();
      // chunk ch is in LDS buffer ch & 1; with two register sets, set ch & 1
      // is free (its chunk is in LDS) and refills with chunk ch + 2, while set
      // (ch + 1) & 1 holds chunk ch + 1 for the other buffer.  Every step
      // issues its loads unconditionally (past the end: the last chunk again,
      // cache hits never stored) so that the compiler counts the loads in
      // flight exactly and waits only for the chunk it stores.
      auto step = [&](int ch, auto par) {
        constexpr int c = decltype(par)::value;
        if (kPre == 2)
          fetch(std::integral_constant<int, c>{}, ks + min(ch + 2, nch - 1) * kBKC);
        else
          fetch(I0{}, ks + min(ch + 1, nch - 1) * kBKC);
        if (ch < nch) compute(c);
        if (ch + 1 < nch) {
          kst = ks + (ch + 1) * kBKC;
          store(std::integral_constant<int, kPre == 2 ? 1 - c : 0>{}, 1 - c);
        }
        __syncthreads();
      };
      for (int ch = 0; ch < nch; ch += 2) {
        step(ch, I0{});
        step(ch + 1, I1{});
      }
    } else {
      fetch(I0{}, ks);
      for (int ch = 0; ch < nch; ++ch) {
        if (ch > 0) __syncthreads();  // the previous chunk's readers are done
        kst = ks + ch * kBKC;
        store(I0{}, 0);
        __syncthreads();
        fetch(I0{}, ks + min(ch + 1, nch - 1) * kBKC);  // unconditional, as above
        compute(0);
      }
      __syncthreads();  // the next segment / the epilogue reuse the LDS
    }
    if (!kKG) break;
  }

  // ---- epilogue: each wave stages one 16-row block at a time as fp32 in its
  // own LDS region (the operand buffers are free after the last barrier) and
  // writes whole row pieces ----
  float *stg = (float *)smem + wave * 16 * kStageStride;
  constexpr int kPieces = NBW * 2;  // 8-column pieces of a wave's staged row
  static_assert(16 * kPieces <= 2 * kWave, "a wave's staged block in two passes");
  float dgrow[MBW][2];
#pragma unroll
  for (int i = 0; i < MBW; ++i) dgrow[i][0] = dgrow[i][1] = 0.f;
#pragma unroll
  for (int i = 0; i < MBW; ++i) {
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) stg[((lane / 16) * 4 + v) * kStageStride + j * 16 + r16] = acc[i][j][v];
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    const int mrow0 = m0 + wm * MBW * 16 + i * 16;
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const int c = lane + c2 * kWave;  // 16 rows x kPieces pieces
      const int rr = c / kPieces, pc = c % kPieces;
      const int m = mrow0 + rr;
      const int n = n0 + wn * NBW * 16 + pc * 8;
      const bool in = c < 16 * kPieces && m < Mt && n < p.Nout;
      float v[8];
      if (c < 16 * kPieces) {
        const f32x4 v0 = *(const f32x4 *)&stg[rr * kStageStride + pc * 8];
        const f32x4 v1 = *(const f32x4 *)&stg[rr * kStageStride + pc * 8 + 4];
        v[0] = v0[0]; v[1] = v0[1]; v[2] = v0[2]; v[3] = v0[3];
        v[4] = v1[0]; v[5] = v1[1]; v[6] = v1[2]; v[7] = v1[3];
      }
      if (EPI == kEpiDW) {
        if (in) {
          bf16x8 o;
#pragma unroll
          for (int q = 0; q < 8; ++q) o[q] = (bf16)v[q];
          *(u32x4 *)((bf16 *)p.Out + (int64_t)e * p.o_estride + (int64_t)m * p.ldo + n) = as_u32x4(o);
        }
      } else if (EPI == kEpiDX) {
        if (in) {
          const int64_t t = p.tok[eC + m];
          // nontemporal, like the weight streams: DU stays in the last-level
          // cache for dW_in (the router's dx reads these 50 MB once, later)
          float *o = (float *)p.Out + t * p.ldo + n;
          __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, (f32x4 *)o);
          __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, (f32x4 *)(o + 4));
        }
      } else if (EPI == kEpiDXR) {
        if (in) {
          const int64_t row = (int64_t)m * p.ldo + n;
          if (!p.dropped[m]) {
            const f32x4 e0 = *(const f32x4 *)(p.dxe + row), e1 = *(const f32x4 *)(p.dxe + row + 4);
            v[0] += e0[0]; v[1] += e0[1]; v[2] += e0[2]; v[3] += e0[3];
            v[4] += e1[0]; v[5] += e1[1]; v[6] += e1[2]; v[7] += e1[3];
          }
          if (p.dyres) {
            const bf16x8 r = as_bf16x8(*(const u32x4 *)(p.dyres + row));
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] += (float)r[q];
          }
          bf16x8 o;
#pragma unroll
          for (int q = 0; q < 8; ++q) o[q] = (bf16)v[q];
          *(u32x4 *)((bf16 *)p.Out + row) = as_u32x4(o);
        }
      } else {  // kEpiDU: du = g z [h > 0], partial <z, h>
        float dot = 0.f;
        if (in) {
          const bf16x8 h = as_bf16x8(*(const u32x4 *)(p.H + (eC + m) * (int64_t)p.Nout + n));
          const float g = p.gmap[eC + m];
          bf16x8 o;
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const float hv = (float)h[q];
            dot += v[q] * hv;
            o[q] = (bf16)(hv > 0.f ? g * v[q] : 0.f);
          }
          *(u32x4 *)((bf16 *)p.Out + (eC + m) * (int64_t)p.Nout + n) = as_u32x4(o);
        }
        // sum the kPieces pieces of each row (consecutive lanes, fixed order)
#pragma unroll
        for (int off = 1; off < kPieces; off <<= 1) dot += __shfl_xor(dot, off, kWave);
        dgrow[i][c2] = dot;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
  }
  if (EPI == kEpiDU) {
    static_assert(kPieces * 16 <= 2 * kWave && (kPieces & (kPieces - 1)) == 0, "row pieces per lane pair");
    // per row: this wave's partial, then the WN waves' partials in order
#pragma unroll
    for (int i = 0; i < MBW; ++i)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const int c = lane + c2 * kWave;
        if (c < 16 * kPieces && c % kPieces == 0) s_dg[wn][wm * MBW * 16 + i * 16 + c / kPieces] = dgrow[i][c2];
      }
    __syncthreads();
    if (tid < BM) {
      const int m = m0 + tid;
      if (m < Mt) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < WN; ++w) s += s_dg[w][tid];
        p.dgpart[(int64_t)p.tok[eC + m] * p.n_tiles + nt] = s;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Weight gradients with a resident operand.  dW_out,e = (G DY)^T H and
// dW_in,e = DU^T X have a short contraction (the expert's kept rows) and a
// large output (d_model x d_ff per expert), so the time goes to writing the
// output and to re-reading operands, not to the MFMAs.  A unit of work is one
// expert, 128 of its d_model columns and a range of its d_ff columns: the
// gathered rows of the d_model operand (g dy or x, through the slot -> token
// map, gate-scaled as in the general kernel) are staged once and then held in
// registers as MFMA operands for the whole unit; the unit walks its d_ff range
// in 64-wide chunks of the expert's H or DU rows (contiguous, double-buffered
// in LDS, the loads two chunks ahead in flight) and writes the output once,
// two chunks at a time as 128 x 128 tiles of whole 256-byte row pieces
// staged through LDS.  The MFMA's row operand is the one that indexes output
// columns, so each lane holds four consecutive outputs of one row.  Per
// output element the contraction runs over the kept rows in steps of 32, in
// order, as in the general kernel.  Four waves and 79 KB of LDS per
// workgroup, two workgroups per CU: while one waits for its stores to drain,
// the other multiplies.  Persistent;
// XCD x takes a contiguous range of units, and the units that share an
// expert's d_ff range are adjacent, so they run side by side and read its H /
// DU rows through one L2.
// ---------------------------------------------------------------------------
constexpr int kWrKmax = 160;          // largest contraction (capacity) this kernel takes
constexpr int kWrR = 128;             // resident (d_model) columns per unit
constexpr int kWrS = 64;              // streamed (d_ff) columns per chunk
constexpr int kWrRS = kWrR + 8;       // LDS row of the resident panel (bf16)
constexpr int kWrSP = kWrS + 8;       // LDS row of a streamed panel (bf16)
constexpr int kWrThreads = 256;       // 2 x 2 waves, each 64 resident x 32 streamed columns
constexpr int kWrWgPerCu = 2;
constexpr int kWrRPer = kWrKmax * (kWrR / 8) / kWrThreads;  // 16-byte resident pieces per thread
constexpr int kWrSPer = kWrKmax * (kWrS / 8) / kWrThreads;  // 16-byte streamed pieces per thread
static_assert(kWrKmax * (kWrS / 8) % kWrThreads == 0 && kWrKmax % 32 == 0, "panel pieces");
static_assert(kWrKmax * kWrRS <= 2 * kWrKmax * kWrSP, "resident panel fits the streamed buffers");

struct WgradArgs {
  int C;
  const int32_t *counts;  // [N] routed tokens per expert (kept = min(count, C))
  const int32_t *tok;     // [N][C] token of each live slot
  const float *gmap;      // [N][C] gate of each live slot (scaled resident rows)
  const bf16 *R;          // resident operand rows: R[token * nres + c], c < nres
  int nres;
  const bf16 *S;          // streamed operand rows: S[(e C + k) * nstr + c], c < nstr
  int nstr;
  bf16 *Out;              // [N] blocks of o_estride elements
  int64_t o_estride;
  int rblocks;            // resident column blocks per expert
  int schunks;            // streamed chunks per expert
  int cpu;                // streamed chunks per unit (the last range may be shorter)
  int splits;             // d_ff ranges per expert
  int nunits;             // N * splits * rblocks
};

// kResRows: the resident operand indexes output rows (dW_out [d][d_ff]),
// else output columns (dW_in [d_ff][d]).  kScale: resident rows are scaled
// by the slot's gate.
template <bool kResRows, bool kScale>
__global__ __launch_bounds__(kWrThreads) void wgrad_res_bf16_kernel(const WgradArgs p) {
  // Two consecutive chunks' tiles are staged side by side and written
  // together as one 128 x 128 tile: whole 256-byte row pieces for both
  // gradients (a chunk alone is 128 rows x 64 columns of dW_out).
  constexpr int kSS = kWrR + 8;
  static_assert(2 * kWrS == kWrR, "a chunk pair spans the resident width");
  __shared__ __attribute__((aligned(16))) bf16 s_str[2][kWrKmax * kWrSP];
  __shared__ __attribute__((aligned(16))) bf16 s_stg[kWrR * kSS];
  bf16 *const s_res = &s_str[0][0];  // resident panel, only while a unit starts

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wr = wave / 2, wc = wave % 2;
  const int nres = p.nres, nstr = p.nstr;
  const int ldo = kResRows ? nstr : nres;

  // resident piece q: contraction row rk[q], column rcol; streamed piece q: row sk[q], column scol
  int rk[kWrRPer], sk[kWrSPer];
  const int rcol = (tid % (kWrR / 8)) * 8, scol = (tid % (kWrS / 8)) * 8;
#pragma unroll
  for (int q = 0; q < kWrRPer; ++q) rk[q] = (tid + q * kWrThreads) / (kWrR / 8);
#pragma unroll
  for (int q = 0; q < kWrSPer; ++q) sk[q] = (tid + q * kWrThreads) / (kWrS / 8);

  const int g8 = gridDim.x / 8, xcd = blockIdx.x % 8;
  const int per = (p.nunits + 7) / 8;
  const int u_end = min(p.nunits, (xcd + 1) * per);
  for (int u = xcd * per + blockIdx.x / 8; u < u_end; u += g8) {
    const int rb = u % p.rblocks, es = u / p.rblocks;
    const int e = es / p.splits, c_lo = (es % p.splits) * p.cpu;
    const int nc = min(p.cpu, p.schunks - c_lo);  // >= 1
    const int live = min(p.counts[e], p.C);
    const int kp = (live + 31) & ~31, nks = kp / 32;
    const int64_t eC = (int64_t)e * p.C;
    const int r0 = rb * kWrR;
    const bf16 *Se = p.S + eC * nstr;

    // Every load and store of the pipeline is unconditional, so that the
    // compiler counts the memory operations in flight exactly and a wait for
    // one chunk's loads never waits for later stores: rows past the live ones
    // re-read a live row (row 0 of the expert, token 0, when it has none) and
    // are stored as zero.
    u32x4 rs[kWrSPer];
    auto fetch_str = [&](int c) {  // chunk c of the expert
      const int col = min(c * kWrS + scol, nstr - 8);
#pragma unroll
      for (int q = 0; q < kWrSPer; ++q)
        rs[q] = *(const u32x4 *)(Se + (int64_t)max(min(sk[q], live - 1), 0) * nstr + col);
    };
    auto store_str = [&](int b) {
#pragma unroll
      for (int q = 0; q < kWrSPer; ++q)
        *(u32x4 *)(&s_str[b][sk[q] * kWrSP + scol]) = sk[q] < live ? rs[q] : u32x4{0, 0, 0, 0};
    };
    bf16x8 res[kWrKmax / 32][4];
    {
      u32x4 rr[kWrRPer];
      float rg[kWrRPer];
      const int col = min(r0 + rcol, nres - 8);
#pragma unroll
      for (int q = 0; q < kWrRPer; ++q) {
        const int64_t slot = eC + max(min(rk[q], live - 1), 0);
        const int32_t t = p.tok[slot];
        rr[q] = *(const u32x4 *)(p.R + (int64_t)(live > 0 ? t : 0) * nres + col);
        if (kScale) rg[q] = p.gmap[slot];
      }
      fetch_str(c_lo);
      __syncthreads();  // the previous unit's last chunk has left the panels
#pragma unroll
      for (int q = 0; q < kWrRPer; ++q) {
        u32x4 v = rr[q];
        if (kScale) {
          bf16x8 b = as_bf16x8(v);
#pragma unroll
          for (int j = 0; j < 8; ++j) b[j] = (bf16)(rg[q] * (float)b[j]);
          v = as_u32x4(b);
        }
        *(u32x4 *)(&s_res[rk[q] * kWrRS + rcol]) = rk[q] < live ? v : u32x4{0, 0, 0, 0};
      }
      __syncthreads();
#pragma unroll
      for (int ks = 0; ks < kWrKmax / 32; ++ks)
        if (ks < nks)
#pragma unroll
          for (int i = 0; i < 4; ++i) res[ks][i] = tr_operand(s_res, kWrRS, ks * 32, wr * 64 + i * 16, lane);
      __syncthreads();  // every wave holds its resident operands before chunk 0 overwrites them
    }
    store_str(0);
    fetch_str(c_lo + min(1, nc - 1));
    __syncthreads();

    // One chunk: multiply, stage its tile into half `kHalf` of the pair
    // (the pair's first chunk waits until every wave has written the
    // previous pair out), move the next chunk into LDS, issue the loads two
    // chunks ahead, and, with kWrite halves, write the pair.  The loop takes
    // chunks in pairs so that every store sits at a fixed place in the code,
    // and the first pair is peeled off it: the loop is entered with the same
    // memory operations in flight as its back edge carries (loads, then the
    // last pair's stores), and a wait for a chunk's loads never includes
    // those stores.
    auto step = [&](auto half_c, auto write_c, const int j) {
      constexpr int kHalf = decltype(half_c)::value, kWrite = decltype(write_c)::value;
      const int b = j & 1;
      f32x4 acc[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kWrKmax / 32; ++ks) {
        if (ks < nks) {
          const bf16x8 s0 = tr_operand(s_str[b], kWrSP, ks * 32, wc * 32, lane);
          const bf16x8 s1 = tr_operand(s_str[b], kWrSP, ks * 32, wc * 32 + 16, lane);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (kResRows) {
              acc[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s0, res[ks][i], acc[i][0], 0, 0, 0);
              acc[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s1, res[ks][i], acc[i][1], 0, 0, 0);
            } else {
              acc[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(res[ks][i], s0, acc[i][0], 0, 0, 0);
              acc[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(res[ks][i], s1, acc[i][1], 0, 0, 0);
            }
          }
        }
      }
      if (kHalf == 0) __syncthreads();  // the previous pair has left the staging area
      // lane: output row (16 x block + lane % 16), four consecutive columns;
      // the chunk's streamed columns are the pair tile's columns (dW_out) or
      // rows (dW_in) kHalf * 64 ...
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
          const int ri = wr * 64 + i * 16, sj = kHalf * kWrS + wc * 32 + jb * 16;
          const int row = (kResRows ? ri : sj) + lane % 16, col = (kResRows ? sj : ri) + (lane / 16) * 4;
          typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
          const bf16x4 o{(bf16)acc[i][jb][0], (bf16)acc[i][jb][1], (bf16)acc[i][jb][2], (bf16)acc[i][jb][3]};
          *(bf16x4 *)(&s_stg[row * kSS + col]) = o;
        }
      // the next chunk into the other buffer (after the last chunk: a copy of
      // it that nothing reads), then loads two chunks ahead
      store_str(b ^ 1);
      fetch_str(c_lo + min(j + 2, nc - 1));
      __syncthreads();
      if (kWrite > 0) {
        // the pair (kWrite chunks), in 16-byte row pieces; pieces past the
        // output's edge write the nearest piece inside it again (same value)
        const int sc = c_lo + j - kHalf;  // the pair's first chunk
        const int row0 = kResRows ? r0 : sc * kWrS, col0 = kResRows ? sc * kWrS : r0;
        constexpr int kRows = kResRows ? kWrR : kWrite * kWrS, kCols = kResRows ? kWrite * kWrS : kWrR;
        const int rlim = min((kResRows ? nres : nstr) - row0, kRows) - 1;
        const int clim = min((kResRows ? nstr : nres) - col0, kCols) - 8;
        bf16 *Ot = p.Out + (int64_t)e * p.o_estride + (int64_t)row0 * ldo + col0;
#pragma unroll
        for (int q = 0; q < kRows * kCols / 8 / kWrThreads; ++q) {
          const int i = tid + q * kWrThreads;
          const int row = min(i / (kCols / 8), rlim), col = min((i % (kCols / 8)) * 8, clim);
          // nontemporal: the gradient is written once, and keeping it out of
          // the last-level cache leaves H and DU there for the other kernels
          __builtin_nontemporal_store(*(const u32x4 *)(&s_stg[row * kSS + col]),
                                      (u32x4 *)(Ot + (int64_t)row * ldo + col));
        }
      }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    int j = 0;
    if (nc >= 2) {
      step(I0{}, I0{}, 0);
      step(I1{}, I2{}, 1);
      for (j = 2; j + 1 < nc; j += 2) {
        step(I0{}, I0{}, j);
        step(I1{}, I2{}, j + 1);
      }
    }
    if (j < nc) step(I0{}, I1{}, j);  // an odd chunk count: the last chunk alone
  }
}

// ---------------------------------------------------------------------------
// fp32 layers: the same products on the vector ALUs.  64 x 64 output tile,
// 256 threads with 4 x 4 outputs each, contraction chunks of 16 staged in LDS
// k-major for both operands (element loads, any layout).
// ---------------------------------------------------------------------------
template <bool AKM, bool AG, bool AS, bool BKM, bool BG, int EPI>
__global__ __launch_bounds__(256) void bwd_gemm_f32_kernel(const BwdArgs<float> p) {
  constexpr int kT = 64, kKs = 16;
  constexpr bool kRaggedM = EPI != kEpiDW;
  __shared__ float sA[kKs][kT + 1], sB[kKs][kT + 1];
  const int64_t id = blockIdx.x;
  if (id >= p.ntiles) return;
  const int e = (int)(id / ((int64_t)p.m_tiles * p.n_tiles));
  const int rem = (int)(id % ((int64_t)p.m_tiles * p.n_tiles));
  const int mt = rem / p.n_tiles, nt = rem % p.n_tiles;
  const int live = min(p.counts[e], p.C);
  const int m0 = mt * kT, n0 = nt * kT;
  const int Mt = kRaggedM ? live : p.M;
  if (m0 >= Mt) return;
  const int Kt = kRaggedM ? p.K : live;
  const int64_t eC = (int64_t)e * p.C;
  const float *Ab = p.A + (AG ? 0 : (int64_t)e * p.a_estride);
  const float *Bb = p.B + (BG ? 0 : (int64_t)e * p.b_estride);
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  // element (r, k) of an operand; r is a row of the tile, k a contraction index
  auto elem = [&](const float *base, int ld, bool km, bool g, bool sc, int r, int rlive, int k) -> float {
    if (km) {
      if (k >= Kt || r >= rlive) return 0.f;
      const int64_t row = g ? (int64_t)p.tok[eC + k] : k;
      const float v = base[row * ld + r];
      return sc ? p.gmap[eC + k] * v : v;
    }
    if (r >= rlive) return 0.f;
    const int64_t row = g ? (int64_t)p.tok[eC + r] : r;
    return base[row * ld + k];
  };
  float acc[4][4] = {};
  for (int k0 = 0; k0 < Kt; k0 += kKs) {
    for (int i = tid; i < kKs * kT; i += 256) {
      const int k = i / kT, r = i % kT;
      sA[k][r] = elem(Ab, p.lda, AKM, AG, AS, m0 + r, Mt, k0 + k);
      sB[k][r] = elem(Bb, p.ldb, BKM, BG, false, n0 + r, p.Nout, k0 + k);
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
    const int m = m0 + ty * 4 + i;
    float dot = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (m >= Mt || n >= p.Nout) continue;
      const float v = acc[i][j];
      if (EPI == kEpiDW) {
        ((float *)p.Out)[(int64_t)e * p.o_estride + (int64_t)m * p.ldo + n] = v;
      } else if (EPI == kEpiDX) {
        ((float *)p.Out)[(int64_t)p.tok[eC + m] * p.ldo + n] = v;
      } else {
        const float h = p.H[(eC + m) * (int64_t)p.Nout + n];
        dot += v * h;
        ((float *)p.Out)[(eC + m) * (int64_t)p.Nout + n] = h > 0.f ? p.gmap[eC + m] * v : 0.f;
      }
    }
    if (EPI == kEpiDU) {
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) dot += __shfl_xor(dot, off, kWave);
      if (tx == 0 && m < Mt) p.dgpart[(int64_t)p.tok[eC + m] * p.n_tiles + nt] = dot;
    }
  }
}

// ---------------------------------------------------------------------------
// Router weight gradient dW_r = sum_t dL/dh_t x_t^T on bf16 MFMA, fp32-exact
// products ("Making Sparse Training Stable": the router stays in fp32): dL/dh
// (fp32) is split while staging into three bf16 planes hi + mid + lo that sum
// to it exactly, x is bf16, so each plane product is exact in fp32 and the
// accumulation sees the terms of an fp32 dot product.  Workgroup (64 experts,
// 128 columns, token range [s ts, (s + 1) ts)) writes its partial sum; both
// operands are k-major (token = contraction) and read with the LDS transpose
// load.  4 waves, each 32 experts x 64 columns.
// ---------------------------------------------------------------------------
constexpr int kWgJ = 64, kWgK = 128, kWgT = 64;

__device__ __forceinline__ void split3(float w, bf16 &hi, bf16 &mid, bf16 &lo) {
  hi = (bf16)w;
  const float r = w - (float)hi;  // exact
  mid = (bf16)r;
  lo = (bf16)(r - (float)mid);  // exact, and representable in bf16
}

__global__ __launch_bounds__(256) void router_wgrad_bf16_kernel(const float *__restrict__ dh,
                                                                const bf16 *__restrict__ x, int64_t T, int N, int d,
                                                                int64_t ts, float *__restrict__ wpart) {
  constexpr int kSA = kWgJ + 8, kSB = kWgK + 8;
  __shared__ __attribute__((aligned(16))) bf16 sA[3 * kWgT * kSA];
  __shared__ __attribute__((aligned(16))) bf16 sB[kWgT * kSB];
  const int j0 = blockIdx.x * kWgJ, k0 = blockIdx.y * kWgK, sp = blockIdx.z;
  const int64_t ta = min<int64_t>(T, (int64_t)sp * ts), tb = min<int64_t>(T, ta + ts);
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wj = wave / 2, wk = wave % 2;
  f32x4 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // staging: dh chunk 64 tokens x 64 experts (pieces of 4 fp32), x chunk 64
  // tokens x 128 columns (pieces of 8 bf16); 4 pieces of each per thread
  float rA[4][4];
  u32x4 rB[4];
  auto fetch = [&](int64_t c) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int pc = tid + q * 256, t = pc / 16;
      const int64_t tt = c + t;
      const int jc = (pc % 16) * 4, kc = (pc % 16) * 8;
#pragma unroll
      for (int e = 0; e < 4; ++e) rA[q][e] = (tt < tb && j0 + jc + e < N) ? dh[tt * N + j0 + jc + e] : 0.f;
      rB[q] = (tt < tb && k0 + kc < d) ? *(const u32x4 *)(x + tt * d + k0 + kc) : u32x4{0, 0, 0, 0};
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int pc = tid + q * 256, t = pc / 16;
      const int jc = (pc % 16) * 4, kc = (pc % 16) * 8;
      bf16 h[4], m[4], l[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) split3(rA[q][e], h[e], m[e], l[e]);
      bf16 *a = sA + t * kSA + jc;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] = h[e];
        a[kWgT * kSA + e] = m[e];
        a[2 * kWgT * kSA + e] = l[e];
      }
      *(u32x4 *)(sB + t * kSB + kc) = rB[q];
    }
  };
  if (ta < tb) fetch(ta);
  for (int64_t c = ta; c < tb; c += kWgT) {
    __syncthreads();  // the previous chunk's readers are done
    store();
    __syncthreads();
    if (c + kWgT < tb) fetch(c + kWgT);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      bf16x8 a[2][3], b[4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int pl = 0; pl < 3; ++pl) a[i][pl] = tr_operand(sA + pl * kWgT * kSA, kSA, s2 * 32, wj * 32 + i * 16, lane);
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) b[jb] = tr_operand(sB, kSB, s2 * 32, wk * 64 + jb * 16, lane);
#pragma unroll
      for (int pl = 0; pl < 3; ++pl)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int jb = 0; jb < 4; ++jb)
            acc[i][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i][pl], b[jb], acc[i][jb], 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      const int k = k0 + wk * 64 + jb * 16 + lane % 16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = j0 + wj * 32 + i * 16 + (lane / 16) * 4 + r;
        if (j < N && k < d) wpart[((int64_t)sp * N + j) * d + k] = acc[i][jb][r];
      }
    }
}

hipError_t launch_router_wgrad_bf16(const float *dh, const void *x, int64_t T, int N, int d, WgradSplit sp,
                                    float *wpart, hipStream_t st) {
  const dim3 g((unsigned)ceil_div(N, kWgJ), (unsigned)ceil_div(d, kWgK), (unsigned)sp.splits);
  router_wgrad_bf16_kernel<<<g, dim3(256), 0, st>>>(dh, (const bf16 *)x, T, N, d, sp.ts, wpart);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The router's part of dx, dx_t += W_r^T dL/dh_t, on bf16 MFMA.  Both fp32
// operands are split exactly into three bf16 planes (hi + mid + lo); the six
// plane products that carry more than 2^-24 of the result -- (hi, hi), (hi,
// mid), (mid, hi), (hi, lo), (lo, hi), (mid, mid) -- are one contraction of
// length 6 N: A' [T][Kp] holds the dL/dh planes in the order hi, hi, mid, hi,
// lo, mid (written by the router kernel), B' [Kp][d] the W_r planes in the
// order hi, mid, hi, lo, hi, mid (rows p N + j; Kp = 6 N rounded up to the
// chunk, padding rows and columns zero).  Each dropped product is below
// 2^-24 of |dL/dh| |W_r| per term, so the sum is fp32-accurate.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_wr_planes_kernel(const float *__restrict__ w_r, int N, int d, int kp,
                                                               bf16 *__restrict__ planes) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)kp * d) return;
  const int row = (int)(i / d), k = (int)(i % d);
  bf16 out = (bf16)0.f;
  if (row < 6 * N) {
    const int pl = row / N, j = row % N;
    bf16 hi, mid, lo;
    split3(w_r[(int64_t)j * d + k], hi, mid, lo);
    static constexpr int kWhich[6] = {0, 1, 0, 2, 0, 1};  // B' order: hi, mid, hi, lo, hi, mid
    out = kWhich[pl] == 0 ? hi : (kWhich[pl] == 1 ? mid : lo);
  }
  planes[i] = out;
}

int router_dx_kp(int N) { return (int)ceil_div(6 * (int64_t)N, kBKC) * kBKC; }

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
namespace {

// Tile shapes: rows of an expert (up to 160) x 256 columns (DZ) or x 128
// columns (DX), 8 waves, a deep pipeline for the products with a long
// contraction; 64 x 256, 4 waves, single-buffered, three workgroups per CU
// for the weight gradients (contraction = an expert's rows, short).
constexpr int kRowMBW = 5, kRowNBW = 4, kRowWM = 2, kRowWN = 4;
constexpr int kDxNBW = 2;  // DX: 128 columns per tile (d_model / 128 tiles per expert)
constexpr int kDxrMBW = 4;  // router dx: 128 token rows per tile (T / 128 x d / 128 tiles, even over the CUs)
constexpr int kWgtMBW = 4, kWgtNBW = 4, kWgtWM = 1, kWgtWN = 4;
constexpr int kBNb = kRowWN * kRowNBW * 16, kBNdx = kRowWN * kDxNBW * 16;

template <typename T_>
BwdArgs<T_> bwd_args(const BwdLaunch &L, const void *A, int64_t ae, int lda, const void *B, int64_t be, int ldb,
                     int M, int Nout, int K, void *Out, int64_t oe, int ldo, int bm, int bn) {
  BwdArgs<T_> a;
  a.C = L.C;
  a.counts = L.counts;
  a.tok = L.tok;
  a.gmap = L.gmap;
  a.A = (const T_ *)A;
  a.a_estride = ae;
  a.lda = lda;
  a.B = (const T_ *)B;
  a.b_estride = be;
  a.ldb = ldb;
  a.M = M;
  a.Nout = Nout;
  a.K = K;
  a.Out = Out;
  a.o_estride = oe;
  a.ldo = ldo;
  a.H = (const T_ *)L.hidden;
  a.dgpart = L.dgpart;
  a.m_tiles = (int)ceil_div(M, bm);
  a.n_tiles = (int)ceil_div(Nout, bn);
  a.ntiles = (int64_t)L.N * a.m_tiles * a.n_tiles;
  return a;
}

template <bool AKM, bool AG, bool AS, bool BKM, bool BG, int EPI>
hipError_t run_bf16(const BwdArgs<bf16> &a, hipStream_t st) {
  if (a.ntiles == 0) return hipSuccess;
  const unsigned grid = (unsigned)(ceil_div(a.ntiles, 8) * 8);
  if constexpr (EPI == kEpiDU)
    bwd_gemm_bf16_kernel<kRowMBW, kRowNBW, kRowWM, kRowWN, AKM, AG, AS, BKM, BG, EPI, 2, 2, 0>
        <<<dim3(grid), dim3(kRowWM * kRowWN * 64), 0, st>>>(a);
  else if constexpr (EPI == kEpiDX)
    bwd_gemm_bf16_kernel<kRowMBW, kDxNBW, kRowWM, kRowWN, AKM, AG, AS, BKM, BG, EPI, 2, 2, 0>
        <<<dim3(grid), dim3(kRowWM * kRowWN * 64), 0, st>>>(a);
  else
    bwd_gemm_bf16_kernel<kWgtMBW, kWgtNBW, kWgtWM, kWgtWN, AKM, AG, AS, BKM, BG, EPI, 1, 1, 3>
        <<<dim3(grid), dim3(kWgtWM * kWgtWN * 64), 0, st>>>(a);
  return hipGetLastError();
}

// Resident operand rows R (through the slot -> token map, width d), streamed
// rows S ([N][C][d_ff]), output [N][d][d_ff] or [N][d_ff][d].
int wgrad_grid_cus() {
  const int cus = device_cus();
  return cus < 8 ? 256 : cus;
}

// Resident operand rows R (through the slot -> token map, width d), streamed
// rows S ([N][C][d_ff]), output [N][d][d_ff] or [N][d_ff][d].  Each expert's
// d_ff chunks are split into `splits` ranges so that the units deal out
// evenly over the workgroups: the split count minimises the chunks (plus
// two for a unit's start) of the busiest workgroup.
WgradArgs wgrad_args(const BwdLaunch &L, const void *R, const void *S, void *Out) {
  WgradArgs a;
  a.C = L.C;
  a.counts = L.counts;
  a.tok = L.tok;
  a.gmap = L.gmap;
  a.R = (const bf16 *)R;
  a.nres = L.d;
  a.S = (const bf16 *)S;
  a.nstr = L.dff;
  a.Out = (bf16 *)Out;
  a.o_estride = (int64_t)L.d * L.dff;
  a.rblocks = (int)ceil_div(L.d, kWrR);
  a.schunks = (int)ceil_div(L.dff, kWrS);
  const int64_t wgs = (int64_t)wgrad_grid_cus() * kWrWgPerCu;
  int best = 1;
  int64_t best_cost = -1;
  for (int sp = 1; sp <= 4 && sp <= a.schunks; ++sp) {
    const int64_t cpu = ceil_div(a.schunks, sp);
    const int64_t units = (int64_t)L.N * a.rblocks * ceil_div(a.schunks, cpu);
    const int64_t cost = ceil_div(units, wgs) * (cpu + 2);
    if (best_cost < 0 || cost < best_cost) best = sp, best_cost = cost;
  }
  a.cpu = (int)ceil_div(a.schunks, best);
  a.splits = (int)ceil_div(a.schunks, a.cpu);  // every range non-empty
  a.nunits = L.N * a.splits * a.rblocks;
  return a;
}

template <bool kResRows, bool kScale>
hipError_t run_wgrad(const WgradArgs &a, hipStream_t st) {
  if (a.nunits == 0) return hipSuccess;
  const int64_t wgs = (int64_t)wgrad_grid_cus() / 8 * 8 * kWrWgPerCu;
  const int64_t grid = std::min<int64_t>(wgs, ceil_div(a.nunits, 8) * 8);
  wgrad_res_bf16_kernel<kResRows, kScale><<<dim3((unsigned)grid), dim3(kWrThreads), 0, st>>>(a);
  return hipGetLastError();
}

template <bool AKM, bool AG, bool AS, bool BKM, bool BG, int EPI>
hipError_t run_f32(const BwdArgs<float> &a, hipStream_t st) {
  if (a.ntiles == 0) return hipSuccess;
  bwd_gemm_f32_kernel<AKM, AG, AS, BKM, BG, EPI><<<dim3((unsigned)a.ntiles), dim3(256), 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router_dx_bf16(const RouterDxArgs &r, hipStream_t st) {
  hipError_t e;
  const int64_t n = (int64_t)r.kp * r.d;
  router_wr_planes_kernel<<<dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, st>>>(r.w_r, r.N, r.d, r.kp,
                                                                                   (bf16 *)r.bplanes);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (r.T == 0) return hipSuccess;
  BwdArgs<bf16> a{};
  a.C = 0;
  a.A = (const bf16 *)r.aplanes;
  a.lda = r.kp;
  a.B = (const bf16 *)r.bplanes;
  a.ldb = r.d;
  a.M = (int)r.T;
  a.Nout = r.d;
  a.K = r.kp;
  a.Out = r.dx;
  a.ldo = r.d;
  a.dxe = r.dxe;
  a.dropped = r.dropped;
  a.dyres = (const bf16 *)r.dyres;
  a.m_tiles = (int)ceil_div(r.T, kRowWM * kDxrMBW * 16);
  a.n_tiles = (int)ceil_div(r.d, kBNdx);
  a.ntiles = (int64_t)a.m_tiles * a.n_tiles;
  const unsigned grid = (unsigned)(ceil_div(a.ntiles, 8) * 8);
  bwd_gemm_bf16_kernel<kDxrMBW, kDxNBW, kRowWM, kRowWN, false, false, false, true, false, kEpiDXR, 2, 2, 0>
      <<<dim3(grid), dim3(kRowWM * kRowWN * 64), 0, st>>>(a);
  return hipGetLastError();
}

int bwd_dz_tiles(int dtype, int dff) { return (int)ceil_div(dff, dtype == kBF16 ? kBNb : 64); }

// The four products, in order: DZ (needs dy, W_out, H), DWO (needs dy, H),
// DX (needs DU), DWI (needs DU, x).
hipError_t launch_bwd_experts(const BwdLaunch &L, hipStream_t st, LaunchMarks marks) {
  auto mark = [&](const char *name) {
    if (marks.fn) marks.fn(marks.ctx, name);
  };
  auto reps = [&]() { return marks.reps ? marks.reps(marks.ctx) : 1; };
  const int d = L.d, f = L.dff, C = L.C;
  const int64_t ein = (int64_t)f * d;  // elements of one expert's W_in / W_out
  const int64_t eh = (int64_t)C * f;   // elements of one expert's H / DU rows
  hipError_t e = hipSuccess;
  auto run = [&](const char *name, auto &&launch) {
    for (int r = reps(); r > 0 && e == hipSuccess; --r) e = launch();
    if (e == hipSuccess) mark(name);
    return e == hipSuccess;
  };
  // Order DZ, dW_out, DX, dW_in: each weight gradient runs right after the
  // kernel that last touched its streamed operand (DZ reads H, DZ writes and
  // DX reads DU), and the weight streams and gradient stores in between are
  // nontemporal, so H and DU are read from the last-level cache.  With no
  // kept rows (C = 0) the row-tiled products launch no tile and the
  // weight-gradient tiles write zeros.
  if (L.dtype == kBF16) {
    const int bm_rows = kRowWM * kRowMBW * 16, bm_w = kWgtWM * kWgtMBW * 16, bn_w = kWgtWN * kWgtNBW * 16;
    const bool resident = C > 0 && C <= kWrKmax && L.T > 0;  // resident-operand weight gradients
    // DZ: A = dy rows through tok (k-contiguous), B = W_out,e [d][d_ff] (k-major)
    auto dz = bwd_args<bf16>(L, L.dy, 0, d, L.w_out, ein, f, C, f, d, L.du, eh, f, bm_rows, kBNb);
    if (!run("bwd_dz", [&] { return run_bf16<false, true, false, true, false, kEpiDU>(dz, st); })) return e;
    // DWO: A = g dy rows through tok (k-major, gate-scaled), B = H,e [rows][d_ff] (k-major)
    auto dwo = bwd_args<bf16>(L, L.dy, 0, d, L.hidden, eh, f, d, f, 0, L.dw_out, ein, f, bm_w, bn_w);
    if (!run("bwd_dw_out", [&] {
          return resident ? run_wgrad<true, true>(wgrad_args(L, L.dy, L.hidden, L.dw_out), st)
                          : run_bf16<true, true, true, true, false, kEpiDW>(dwo, st);
        }))
      return e;
    // DX: A = DU,e [rows][d_ff] (k-contiguous), B = W_in,e [d_ff][d] (k-major)
    auto dx = bwd_args<bf16>(L, L.du, eh, f, L.w_in, ein, d, C, d, f, L.dxe, 0, d, bm_rows, kBNdx);
    if (!run("bwd_dx", [&] { return run_bf16<false, false, false, true, false, kEpiDX>(dx, st); })) return e;
    // DWI: A = DU,e [rows][d_ff] (k-major), B = x rows through tok (k-major)
    auto dwi = bwd_args<bf16>(L, L.du, eh, f, L.x, 0, d, f, d, 0, L.dw_in, ein, d, bm_w, bn_w);
    if (!run("bwd_dw_in", [&] {
          return resident ? run_wgrad<false, false>(wgrad_args(L, L.x, L.du, L.dw_in), st)
                          : run_bf16<true, false, false, true, true, kEpiDW>(dwi, st);
        }))
      return e;
    return hipSuccess;
  }
  auto dz = bwd_args<float>(L, L.dy, 0, d, L.w_out, ein, f, C, f, d, L.du, eh, f, 64, 64);
  if (!run("bwd_dz", [&] { return run_f32<false, true, false, true, false, kEpiDU>(dz, st); })) return e;
  auto dwo = bwd_args<float>(L, L.dy, 0, d, L.hidden, eh, f, d, f, 0, L.dw_out, ein, f, 64, 64);
  if (!run("bwd_dw_out", [&] { return run_f32<true, true, true, true, false, kEpiDW>(dwo, st); })) return e;
  auto dx = bwd_args<float>(L, L.du, eh, f, L.w_in, ein, d, C, d, f, L.dxe, 0, d, 64, 64);
  if (!run("bwd_dx", [&] { return run_f32<false, false, false, true, false, kEpiDX>(dx, st); })) return e;
  auto dwi = bwd_args<float>(L, L.du, eh, f, L.x, 0, d, f, d, 0, L.dw_in, ein, d, 64, 64);
  if (!run("bwd_dw_in", [&] { return run_f32<true, false, false, true, true, kEpiDW>(dwi, st); })) return e;
  return hipSuccess;
}

}  // namespace smx
