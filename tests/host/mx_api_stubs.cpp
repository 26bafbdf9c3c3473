// Stub kernel launchers for the host-only sanitizer build of the libmx C ABI:
// mx_api.cpp and mx_grid.cpp link against these instead of the HIP kernels.
// Each launcher records its call and returns the status the driver selected;
// C accessors let the C driver (mx_api_driver.c) read what was recorded.
#include "mx_kernels.h"

namespace {
int g_calls = 0;
hipError_t g_result = hipSuccess;
mx::CastArgs g_cast{};
mx::NvArgs g_nv{};
mx::RqArgs g_rq{};
uint32_t g_nblocks = 0;

hipError_t record() {
  ++g_calls;
  return g_result;
}
}  // namespace

namespace mx {
hipError_t launch_cast(bool, int, int, int, const CastArgs& a, uint32_t nb, hipStream_t) {
  g_cast = a;
  g_nblocks = nb;
  return record();
}
hipError_t launch_cast_2d(bool, int, int, int, const CastArgs& a, uint32_t nb, hipStream_t) {
  g_cast = a;
  g_nblocks = nb;
  return record();
}
hipError_t launch_cast_sr(bool, int, int, int, bool, const CastArgs& a, uint32_t nb, hipStream_t) {
  g_cast = a;
  g_nblocks = nb;
  return record();
}
hipError_t launch_nvfp4_global(bool, const void*, int64_t, int64_t, float*, hipStream_t) { return record(); }
hipError_t launch_nvfp4_cast(bool, int, const NvArgs& a, uint32_t nb, hipStream_t) {
  g_nv = a;
  g_nblocks = nb;
  return record();
}
hipError_t launch_nvfp4_dequant(bool, const uint8_t*, const uint8_t*, const float*, void*, int64_t, int64_t,
                                hipStream_t) {
  return record();
}
hipError_t launch_requant(int, int, int, const RqArgs& a, hipStream_t) {
  g_rq = a;
  return record();
}
hipError_t launch_copy_nt(const void*, void*, int64_t, hipStream_t) { return record(); }
hipError_t launch_dequant(int, bool, const uint8_t*, const uint8_t*, void*, int64_t, int64_t, hipStream_t) {
  return record();
}
}  // namespace mx

extern "C" {
int stub_calls(void) { return g_calls; }
void stub_fail_launches(int fail) { g_result = fail ? hipErrorInvalidValue : hipSuccess; }
unsigned stub_nblocks(void) { return g_nblocks; }
unsigned stub_cast_flags(void) { return g_cast.flags; }
unsigned stub_cast_tiles_r(void) { return g_cast.tiles_r; }
unsigned stub_cast_tiles_c(void) { return g_cast.tiles_c; }
long long stub_cast_cols(void) { return g_cast.cols; }
int stub_cast_has_row_codes(void) { return g_cast.row_codes != nullptr; }
unsigned stub_cast_seed_lo(void) { return g_cast.seed_lo; }
unsigned stub_cast_seed_hi(void) { return g_cast.seed_hi; }
unsigned stub_nv_flags(void) { return g_nv.flags; }
unsigned stub_rq_tiles_r(void) { return g_rq.tiles_r; }
unsigned stub_rq_tiles_c(void) { return g_rq.tiles_c; }
unsigned stub_rq_total(void) { return g_rq.total_tiles; }
unsigned stub_rq_flags(void) { return g_rq.flags; }
// the flag values the C driver checks
unsigned stub_flag(int which) {
  switch (which) {
    case 0: return mx::kRowScaleDword;
    case 1: return mx::kColScaleDword;
    case 2: return mx::kStaggerStrips;
    case 3: return mx::kRowScaleQword;
    case 4: return mx::kNvMarkedAmax;
    case 5: return mx::kRqScaleWords;
    default: return mx::kRqXcdRows;
  }
}
}
