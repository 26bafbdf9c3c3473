// The MX cast with round-to-nearest-even and 1x32 blocks: dispatch. The
// kernels are templates in mx_cast_impl.h; the launch geometry is in mx_grid.cpp.
#include "mx_cast_impl.h"

namespace mx {

hipError_t launch_cast(bool in_bf16, int fmt, int mode, int axis, const CastArgs& a,
                       uint32_t nblocks, hipStream_t s) {
  return launch_variant<kRne, false>(in_bf16, fmt, mode, axis, a, nblocks, s);
}

}  // namespace mx
