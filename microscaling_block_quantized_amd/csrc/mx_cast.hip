// The MX cast with round-to-nearest-even and 1x32 blocks: launch geometry and
// dispatch. The kernels are templates in mx_cast_impl.h.
#include "mx_cast_impl.h"

namespace mx {

CastGrid cast_grid(int64_t batch, int64_t rows, int64_t cols, bool row_stream) {
  CastGrid g;
  g.tiles_r = (rows + kTileR - 1) / kTileR;
  g.tiles_c = (cols + kTileC - 1) / kTileC;
  if (row_stream) {
    const int64_t per_block = int64_t(kRowThreads / 64) * 64 * kRowSteps * 8;   // elements (BF16 bound)
    g.blocks = (batch * rows * cols + per_block - 1) / per_block * 2;           // FP32 needs twice as many
  } else {
    g.blocks = batch * g.tiles_r * g.tiles_c;
  }
  return g;
}

hipError_t launch_cast(bool in_bf16, int fmt, int mode, int axis, const CastArgs& a,
                       uint32_t nblocks, hipStream_t s) {
  return launch_variant<kRne, false>(in_bf16, fmt, mode, axis, a, nblocks, s);
}

}  // namespace mx
