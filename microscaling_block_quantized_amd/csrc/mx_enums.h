// Enumerations and launch geometry shared by the host-side C ABI
// (mx_api.cpp, mx_grid.cpp) and the kernels. Host-only code may include this
// header without any device code.
#pragma once
#include <stdint.h>

namespace mx {

enum Fmt : int { kE4M3 = 0, kE5M2 = 1, kE2M1 = 2, kE2M3 = 3, kE3M2 = 4, kInt8 = 5 };
enum Mode : int { kFloor = 0, kRoundUp = 1 };
enum Axis : int { kRow = 1, kCol = 2, kBoth = 3 };

// Tiled casts (MX and NVFP4): a workgroup of 8 waves owns a 128-row x
// 256-column tile, waves stacked 4 along rows (32 rows each) and 2 along
// columns (128 each).
constexpr int kWaveRows = 4;
constexpr int kWaveCols = 2;
constexpr int kTileR = 32 * kWaveRows;       // 128
constexpr int kTileC = 128 * kWaveCols;      // 256
constexpr int kTileCNarrow = 64 * kWaveCols; // 128: the FP32 column-only cast with stochastic rounding
constexpr int kThreads = 64 * kWaveRows * kWaveCols;
// Row-only MX cast: 256-thread workgroups, kRowSteps 1 KiB steps per wave.
constexpr int kRowThreads = 256;
constexpr int kRowSteps = 2;
// Non-temporal copy: one 16-byte chunk per thread.
constexpr int kCopyThreads = 256;

}  // namespace mx
