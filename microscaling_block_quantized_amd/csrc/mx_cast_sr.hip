// The MX cast with stochastic rounding, 1x32 or 32x32 blocks (kernels in
// mx_cast_impl.h, the rounding rule and its random bits in mx_sr.h).
#include "mx_cast_impl.h"

namespace mx {

hipError_t launch_cast_sr(bool in_bf16, int fmt, int mode, int axis, bool blocks_2d, const CastArgs& a,
                          uint32_t nblocks, hipStream_t s) {
  return blocks_2d ? launch_variant<kSr, true>(in_bf16, fmt, mode, axis, a, nblocks, s)
                   : launch_variant<kSr, false>(in_bf16, fmt, mode, axis, a, nblocks, s);
}

}  // namespace mx
