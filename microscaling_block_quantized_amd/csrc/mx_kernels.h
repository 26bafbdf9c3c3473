// Internal interface between the C ABI (mx_api.cpp) and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_enums.h"

namespace mx {

template <typename T>
struct Same {
  using type = T;
};

// Launches kernel k and returns the status of this launch itself, as
// hipLaunchKernel reports it, so an error left behind by an unrelated earlier
// call is neither reported as this launch's nor cleared. Arguments convert to
// the kernel's parameter types.
template <typename... P>
hipError_t launch_kernel(void (*k)(P...), dim3 grid, dim3 block, hipStream_t s, typename Same<P>::type... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, argv, 0, s);
}

// One quantize launch over a dense [batch][rows][cols] tensor.
struct CastArgs {
  const void* x;          // BF16 or FP32 elements
  void* row_codes;        // [batch][rows][cols * bits / 8] or null
  uint8_t* row_scales;    // [batch][rows][cols/32] (32x32 blocks: [batch][rows/32][cols/32]) or null
  void* col_codes;        // [batch][cols][rows * bits / 8] or null
  uint8_t* col_scales;    // [batch][cols][rows/32] (32x32 blocks: [batch][cols/32][rows/32]) or null
  int64_t rows, cols;     // per batch slice
  int64_t elements;       // batch * rows * cols
  uint32_t tiles_r, tiles_c;
  uint32_t flags;         // kRowScaleDword / kColScaleDword / kStaggerStrips / kRowScaleQword
  uint32_t seed_lo, seed_hi;   // Philox key of stochastic rounding
};

// A tile's 4 scale bytes per row (column) may be stored as one dword: the
// plane's row pitch is a multiple of 4 bytes and its base is 4-byte aligned.
// With 32x32 blocks the pitches are C/32 (row copy) and R/32 (column copy).
constexpr uint32_t kRowScaleDword = 1u;
constexpr uint32_t kColScaleDword = 2u;
constexpr uint32_t kNvMarkedAmax = 4u;   // NVFP4 cast: global_scale holds marked maxima
// Tiled MX cast: rotate each XCD strip's walk over the tile rows (tile_coords).
// Set by the host when the column plane's pitch is a multiple of 4 KiB.
constexpr uint32_t kStaggerStrips = 8u;
// Tiled MX cast with both copies and 1x32 blocks: every tile is 256 columns
// wide (cols % 256 == 0) and the row-scale plane is 8-byte aligned, so a tile
// row's 8 row-scale bytes can be stored as one 8-byte word.
constexpr uint32_t kRowScaleQword = 16u;
// NVFP4 cast with both copies: cols % 256 == 0 and the row-scale plane 16-byte
// aligned, so a tile row's 16 row-scale bytes can be stored as one 16-byte word.
constexpr uint32_t kNvRowScaleWords = 32u;

struct CastGrid {
  int64_t tiles_r, tiles_c, blocks;
};

// Launch geometry; `blocks` bounds the workgroup count of the chosen kernel:
// the row-only stream kernel (row_stream) or the tiled one.
// narrow: the FP32 column-only cast with stochastic rounding (kTileCNarrow-column tiles)
CastGrid cast_grid(int64_t batch, int64_t rows, int64_t cols, bool row_stream, bool narrow = false);
// Round-to-nearest-even, 1x32 blocks.
hipError_t launch_cast(bool in_bf16, int fmt, int mode, int axis, const CastArgs& a,
                       uint32_t nblocks, hipStream_t s);
// Round-to-nearest-even, 32x32 blocks (always the tiled kernel).
hipError_t launch_cast_2d(bool in_bf16, int fmt, int mode, int axis, const CastArgs& a,
                          uint32_t nblocks, hipStream_t s);
// Stochastic rounding, 1x32 or 32x32 blocks.
hipError_t launch_cast_sr(bool in_bf16, int fmt, int mode, int axis, bool blocks_2d, const CastArgs& a,
                          uint32_t nblocks, hipStream_t s);

// One NVFP4 cast over a dense [batch][rows][cols] tensor (mx_nvfp4.hip): E2M1
// codes two per byte, UE4M3 scales per 16 elements, FP32 global scale per slice.
struct NvArgs {
  const void* x;
  void* row_codes;             // [batch][rows][cols/2] or null
  uint8_t* row_scales;         // [batch][rows][cols/16] or null
  void* col_codes;             // [batch][cols][rows/2] or null
  uint8_t* col_scales;         // [batch][cols][rows/16] or null
  float* global_scale;         // [batch]; with kNvMarkedAmax, raw marked maxima that the cast turns into g
  int64_t rows, cols;
  uint32_t tiles_r, tiles_c;
  uint32_t flags;              // kRowScaleDword: cols % 64 == 0; kColScaleDword: rows % 64 == 0;
                               // kNvMarkedAmax; kNvRowScaleWords
};

// gs[b] = (largest finite |x| of slice b) as FP32 bits with the sign bit set
// (two launches); the cast, given kNvMarkedAmax, turns it into g = amax / 2688.
hipError_t launch_nvfp4_global(bool in_bf16, const void* x, int64_t batch, int64_t slice_elems, float* gs,
                               hipStream_t s);
hipError_t launch_nvfp4_cast(bool in_bf16, int axis, const NvArgs& a, uint32_t nblocks, hipStream_t s);
hipError_t launch_nvfp4_dequant(bool out_bf16, const uint8_t* codes, const uint8_t* scales, const float* gs,
                                void* y, int64_t nblocks, int64_t blocks_per_slice, hipStream_t s);

// FP4-in-FP8 requantization of one MXFP4 plane [batch][rows][cols] (codes two per
// byte, E8M0 scales per 32 elements along cols) into E4M3 with one FP32 scale
// per 128x128 block (mx_requant.hip).
struct RqArgs {
  const uint8_t* codes;        // [batch][rows][cols/2]   (source kFromMx)
  const uint8_t* scales;       // [batch][rows][cols/32]  (source kFromMx)
  const void* x;               // [batch][rows][cols] BF16 / FP32 master weights (kFromBf16 / kFromF32)
  uint8_t* out_codes;          // the MXFP4 plane cast from x, or null
  uint8_t* out_scales;
  uint8_t* fp8;                // [batch][rows][cols] or null
  float* block_scale;          // [batch][R'][C'] or null (R' = ceil(rows/128), C' = ceil(cols/128))
  uint8_t* fp8_t;              // [batch][cols][rows] or null
  float* block_scale_t;        // [batch][C'][R'] or null
  uint8_t* spread;             // [batch][R'][C'] or null
  int64_t rows, cols;
  uint32_t tiles_r, tiles_c;   // 128-row x 256-column tiles per slice
  uint32_t total_tiles;        // batch * tiles_r * tiles_c: one workgroup each
  uint32_t flags;              // kRqScaleWords
};
// Requantization from an MXFP4 plane, with both copies, cols % 256 == 0
// (every tile full width) and a 4-byte-aligned scale plane: each thread loads
// one dword of its tile's scales (tile row t / 2, bytes 4 (t & 1) .. +3) into LDS.
constexpr uint32_t kRqScaleWords = 1u;
// XCD x (workgroup % 8) takes tile rows x, x + 8, ... (all tiles of each), so
// each 128-byte line of the scale plane is fetched into one XCD's L2 instead
// of all eight. Set when batch * tiles_r is a multiple of 8.
constexpr uint32_t kRqXcdRows = 2u;
enum RqSource : int { kFromMx = 0, kFromBf16 = 1, kFromF32 = 2 };
// mode: the MXFP4 scale rule (kFloor / kRoundUp) when casting from x.
hipError_t launch_requant(int src, int mode, int axis, const RqArgs& a, hipStream_t s);

// Plain 16-byte non-temporal copy (mx_copy.hip); bytes % 16 == 0, 16-byte aligned.
int64_t copy_blocks(int64_t bytes);
hipError_t launch_copy_nt(const void* src, void* dst, int64_t bytes, hipStream_t s);

// Dequantize n elements (n % 32 == 0) laid out with blocks along the flat order,
// or, when cols > 0, with 32x32 blocks over rows of `cols` elements (scale
// of element (r, c): scales[(r / 32) * (cols / 32) + c / 32], r counting
// across the batch).
hipError_t launch_dequant(int fmt, bool out_bf16, const uint8_t* codes, const uint8_t* scales,
                          void* y, int64_t n, int64_t cols, hipStream_t s);

}  // namespace mx
