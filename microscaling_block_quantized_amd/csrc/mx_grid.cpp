// Launch geometry of the casts and the copy (host code).
#include "mx_kernels.h"

namespace mx {

CastGrid cast_grid(int64_t batch, int64_t rows, int64_t cols, bool row_stream, bool narrow) {
  CastGrid g;
  const int64_t tc = narrow ? kTileCNarrow : kTileC;
  g.tiles_r = (rows + kTileR - 1) / kTileR;
  g.tiles_c = (cols + tc - 1) / tc;
  if (row_stream) {
    const int64_t per_block = int64_t(kRowThreads / 64) * 64 * kRowSteps * 8;   // elements (BF16 bound)
    g.blocks = (batch * rows * cols + per_block - 1) / per_block * 2;           // FP32 needs twice as many
  } else {
    g.blocks = batch * g.tiles_r * g.tiles_c;
  }
  return g;
}

int64_t copy_blocks(int64_t bytes) { return (bytes / 16 + kCopyThreads - 1) / kCopyThreads; }

}  // namespace mx
