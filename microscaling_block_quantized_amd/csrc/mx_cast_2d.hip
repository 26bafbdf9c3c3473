// The MX cast with 32x32 blocks and round-to-nearest-even (kernels in
// mx_cast_impl.h).
#include "mx_cast_impl.h"

namespace mx {

hipError_t launch_cast_2d(bool in_bf16, int fmt, int mode, int axis, const CastArgs& a,
                          uint32_t nblocks, hipStream_t s) {
  return launch_variant<kRne, true>(in_bf16, fmt, mode, axis, a, nblocks, s);
}

}  // namespace mx
