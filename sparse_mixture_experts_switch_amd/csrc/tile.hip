// Expert weights in the tiled layout: each expert matrix ([rows][cols], the
// contraction dimension cols contiguous, as W_in [d_ff][d_model] and W_out
// [d_model][d_ff] are stored row-major) split into 16-row x 32-column blocks,
// the blocks in row-major order, and each block stored as the operand of
// v_mfma_f32_16x16x32_bf16: 64 lanes x 8 bf16, lane l holding row l % 16 and
// columns 8 (l / 16) .. 8 (l / 16) + 7 of the block.  A wave then loads one
// block of weights with one contiguous 1 KB access instead of 16 pieces from
// 16 rows.  The layout only moves values: the expert FFN reads every weight
// into the same operand lane either way, so results are identical.
//
// This file converts between the two layouts; it is a one-off conversion of
// the parameters (when weights are loaded or updated), not part of a layer
// call.  One thread per 16-byte piece; the tiled side is written (or read)
// contiguously, the row-major side in 16-byte pieces of 16 rows.

#include "common.h"
#include "launch.h"

#include <algorithm>

namespace smx {

constexpr int kTileThreads = 256;

template <bool kToTiled>
__global__ __launch_bounds__(kTileThreads) void tile_weights_kernel(const u32x4 *__restrict__ src,
                                                                    u32x4 *__restrict__ dst, int64_t pieces,
                                                                    int rows, int cols) {
  const int64_t per = (int64_t)rows * cols / 8;  // pieces per matrix
  const int kb = cols / 32;                      // column blocks per row block
  for (int64_t i = (int64_t)blockIdx.x * kTileThreads + threadIdx.x; i < pieces;
       i += (int64_t)gridDim.x * kTileThreads) {
    // i: piece of the tiled layout = (matrix m, block b, lane l)
    const int64_t m = i / per, q = i % per;
    const int64_t b = q / 64;
    const int l = (int)(q % 64);
    const int64_t r = (b / kb) * 16 + l % 16;
    const int64_t c = (b % kb) * 32 + (l / 16) * 8;
    const int64_t j = ((m * rows + r) * cols + c) / 8;  // the same piece, row-major
    if (kToTiled)
      dst[i] = src[j];
    else
      dst[j] = src[i];
  }
}

hipError_t launch_tile_weights(const TileArgs &a, hipStream_t st) {
  const int64_t pieces = a.count * a.rows * a.cols / 8;
  if (pieces == 0) return hipSuccess;
  const int64_t want = ceil_div(pieces, kTileThreads);
  const unsigned grid = (unsigned)std::min<int64_t>(want, (int64_t)device_cus() * 16);
  if (a.to_tiled)
    tile_weights_kernel<true><<<dim3(grid), dim3(kTileThreads), 0, st>>>((const u32x4 *)a.src, (u32x4 *)a.dst,
                                                                          pieces, a.rows, a.cols);
  else
    tile_weights_kernel<false><<<dim3(grid), dim3(kTileThreads), 0, st>>>((const u32x4 *)a.src, (u32x4 *)a.dst,
                                                                           pieces, a.rows, a.cols);
  return hipGetLastError();
}

}  // namespace smx
