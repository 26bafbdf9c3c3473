// Internal interface between the C ABI (mx_api.cpp) and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_device.h"

namespace mx {

// One quantize launch over a dense [batch][rows][cols] tensor.
struct CastArgs {
  const void* x;          // BF16 or FP32 elements
  void* row_codes;        // [batch][rows][cols] (E2M1: [..][cols/2]) or null
  uint8_t* row_scales;    // [batch][rows][cols/32] or null
  void* col_codes;        // [batch][cols][rows] (E2M1: [..][rows/2]) or null
  uint8_t* col_scales;    // [batch][cols][rows/32] or null
  int64_t rows, cols;     // per batch slice
  int64_t elements;       // batch * rows * cols
  uint32_t tiles_r, tiles_c;
  uint32_t flags;         // kRowScaleDword / kColScaleDword
};

// A tile's 4 scale bytes per row (column) may be stored as one dword: the
// plane's row pitch is a multiple of 4 bytes and its base is 4-byte aligned.
constexpr uint32_t kRowScaleDword = 1u;
constexpr uint32_t kColScaleDword = 2u;

struct CastGrid {
  int64_t tiles_r, tiles_c, blocks;
};

// Launch geometry; `blocks` bounds the workgroup count of the chosen kernel.
CastGrid cast_grid(int64_t batch, int64_t rows, int64_t cols, int axis);
hipError_t launch_cast(bool in_bf16, int fmt, int mode, int axis, const CastArgs& a,
                       uint32_t nblocks, hipStream_t s);

// Dequantize n elements (n % 32 == 0) laid out with blocks along the flat order.
hipError_t launch_dequant(int fmt, bool out_bf16, const uint8_t* codes, const uint8_t* scales,
                          void* y, int64_t n, hipStream_t s);

}  // namespace mx
