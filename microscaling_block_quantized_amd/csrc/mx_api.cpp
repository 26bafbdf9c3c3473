// C ABI of libmx: argument validation, plane-size arithmetic and kernel dispatch.
// Every argument check runs before the first HIP call, so argument errors are
// reported synchronously and without touching a device.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "../../include/libmx.h"
#include "mx_kernels.h"

namespace {

constexpr int64_t kBlock = 32;
constexpr int64_t kMaxGrid = (int64_t(1) << 31) - 1;

bool valid_fmt(int f) {
  return f == MX_E4M3 || f == MX_E5M2 || f == MX_E2M1 || f == MX_E2M3 || f == MX_E3M2 || f == MX_INT8;
}
bool valid_mode(int m) { return m == MX_SCALE_FLOOR || m == MX_SCALE_ROUNDUP; }
bool valid_dtype(int d) { return d == MX_F32 || d == MX_BF16; }
bool valid_axis(int a) { return a == MX_AXIS_ROW || a == MX_AXIS_COL || a == MX_AXIS_BOTH; }
bool valid_rounding(int r) { return r == MX_ROUND_NEAREST_EVEN || r == MX_ROUND_STOCHASTIC; }
bool valid_block(int b) { return b == MX_BLOCK_1X32 || b == MX_BLOCK_32X32; }

int code_bits(int fmt) { return fmt == MX_E2M1 ? 4 : (fmt == MX_E2M3 || fmt == MX_E3M2) ? 6 : 8; }
// dequantize reads 16 codes per thread: 16, 12 or 8 bytes
uintptr_t dequant_code_align(int fmt) { return fmt == MX_E2M1 ? 8 : code_bits(fmt) == 6 ? 4 : 16; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
Range range_of(const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + uintptr_t(bytes)};
}
bool overlap(const Range& a, const Range& b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

// Element count, or -1 if an extent is non-positive or the product overflows.
int64_t elements(const mx_shape& s) {
  if (s.batch < 1 || s.rows < 1 || s.cols < 1) return -1;
  const int64_t lim = INT64_C(1) << 56;
  if (s.batch > lim || s.rows > lim || s.cols > lim) return -1;
  if (s.rows > lim / s.cols) return -1;
  const int64_t rc = s.rows * s.cols;
  if (s.batch > lim / rc) return -1;
  return s.batch * rc;
}

}  // namespace

extern "C" {

int mx_version(void) { return 10700; }

const char* mx_strerror(int err) {
  switch (err) {
    case MX_OK: return "ok";
    case MX_ERR_NULL: return "a required pointer is NULL, or a pointer of an unused axis is not";
    case MX_ERR_SHAPE: return "invalid shape: extents must be >= 1 and blocked extents multiples of the block";
    case MX_ERR_ALIGN: return "a data pointer is not aligned as required";
    case MX_ERR_ENUM: return "unknown format, scale mode, dtype or axis";
    case MX_ERR_ALIAS: return "input and output buffers overlap";
    case MX_ERR_TOO_LARGE: return "tensor too large for one launch";
    case MX_ERR_LAUNCH: return "HIP kernel launch failed";
    default: return "unknown libmx error";
  }
}

int mx_plane_bytes(mx_fmt fmt, mx_shape s, mx_axis axis, size_t* code_bytes, size_t* scale_bytes) {
  if (!valid_fmt(fmt) || !valid_axis(axis)) return MX_ERR_ENUM;
  if (code_bytes == nullptr || scale_bytes == nullptr) return MX_ERR_NULL;
  const int64_t n = elements(s);
  const bool row = (axis & MX_AXIS_ROW) != 0, col = (axis & MX_AXIS_COL) != 0;
  if (n < 0 || (row && s.cols % kBlock != 0) || (col && s.rows % kBlock != 0)) return MX_ERR_SHAPE;
  const int64_t planes = (row ? 1 : 0) + (col ? 1 : 0);
  // n is a multiple of 32 (one blocked extent is), so both divisions are exact
  *code_bytes = size_t(planes * (n / 8 * code_bits(fmt)));
  *scale_bytes = size_t(planes * (n / kBlock));
  return MX_OK;
}

int mx_quantize(const void* x, mx_dtype x_dtype, mx_shape s, mx_fmt fmt, mx_scale_mode mode,
                mx_axis axis, void* row_codes, uint8_t* row_scales, void* col_codes,
                uint8_t* col_scales, void* stream) {
  return mx_quantize_ex(x, x_dtype, s, fmt, mode, axis, nullptr, row_codes, row_scales, col_codes, col_scales,
                        stream);
}

int mx_quantize_ex(const void* x, mx_dtype x_dtype, mx_shape s, mx_fmt fmt, mx_scale_mode mode,
                   mx_axis axis, const mx_quant_opts* opts, void* row_codes, uint8_t* row_scales,
                   void* col_codes, uint8_t* col_scales, void* stream) {
  // The enum fields of a caller's options struct are read as the ints a C
  // caller stored (any value is legal there; loading an out-of-range value as
  // a C++ enum would not be).
  static_assert(sizeof(mx_rounding) == sizeof(int) && sizeof(mx_block) == sizeof(int), "enum fields are ints");
  int rounding = MX_ROUND_NEAREST_EVEN, block = MX_BLOCK_1X32;
  uint64_t seed = 0;
  if (opts != nullptr) {
    std::memcpy(&rounding, &opts->rounding, sizeof(int));
    std::memcpy(&block, &opts->block, sizeof(int));
    seed = opts->seed;
  }
  if (!valid_fmt(fmt) || !valid_mode(mode) || !valid_dtype(x_dtype) || !valid_axis(axis) ||
      !valid_rounding(rounding) || !valid_block(block))
    return MX_ERR_ENUM;
  const bool b2d = block == MX_BLOCK_32X32;
  const bool sr = rounding == MX_ROUND_STOCHASTIC;
  const bool want_row = (axis & MX_AXIS_ROW) != 0;
  const bool want_col = (axis & MX_AXIS_COL) != 0;
  if (x == nullptr) return MX_ERR_NULL;
  if (want_row != (row_codes != nullptr) || want_row != (row_scales != nullptr)) return MX_ERR_NULL;
  if (want_col != (col_codes != nullptr) || want_col != (col_scales != nullptr)) return MX_ERR_NULL;
  const int64_t n = elements(s);
  // blocked extents are multiples of 32; a column-only cast with 1x32 blocks
  // blocks no run along cols, which then needs only whole 16-byte row vectors
  const int64_t col_mult = (want_row || b2d) ? kBlock : (x_dtype == MX_BF16 ? 8 : 4);
  if (n < 0 || s.cols % col_mult != 0) return MX_ERR_SHAPE;
  if ((want_col || b2d) && s.rows % kBlock != 0) return MX_ERR_SHAPE;
  if (!aligned(x, 16) || (want_row && !aligned(row_codes, 16)) || (want_col && !aligned(col_codes, 16)))
    return MX_ERR_ALIGN;

  const int64_t in_bytes = n * (x_dtype == MX_BF16 ? 2 : 4);
  const int64_t cbytes = n / 8 * code_bits(fmt);
  const int64_t sbytes = n / (b2d ? kBlock * kBlock : kBlock);
  Range rs[5];
  int nr = 0;
  rs[nr++] = range_of(x, in_bytes);
  if (want_row) { rs[nr++] = range_of(row_codes, cbytes); rs[nr++] = range_of(row_scales, sbytes); }
  if (want_col) { rs[nr++] = range_of(col_codes, cbytes); rs[nr++] = range_of(col_scales, sbytes); }
  for (int i = 0; i < nr; ++i)
    for (int j = i + 1; j < nr; ++j)
      if (overlap(rs[i], rs[j])) return MX_ERR_ALIAS;

  const bool row_stream = axis == MX_AXIS_ROW && !b2d;
  // the FP32 column-only stochastic-rounding kernel runs narrow tiles
  const bool narrow = sr && !b2d && x_dtype == MX_F32 && axis == MX_AXIS_COL;
  const mx::CastGrid g = mx::cast_grid(s.batch, s.rows, s.cols, row_stream, narrow);
  if (g.blocks > kMaxGrid) return MX_ERR_TOO_LARGE;
  // per-thread offsets inside a tile are 32-bit: 128 rows of FP32 and 256 column-plane rows
  if (s.cols >= (INT64_C(1) << 22) || (want_col && s.rows >= (INT64_C(1) << 23))) return MX_ERR_TOO_LARGE;

  mx::CastArgs a;
  a.x = x;
  a.row_codes = row_codes;
  a.row_scales = row_scales;
  a.col_codes = col_codes;
  a.col_scales = col_scales;
  a.rows = s.rows;
  a.cols = s.cols;
  a.elements = n;
  a.tiles_r = uint32_t(g.tiles_r);
  a.tiles_c = uint32_t(g.tiles_c);
  a.flags = 0;
  a.seed_lo = uint32_t(seed);
  a.seed_hi = uint32_t(seed >> 32);
  // the row-only kernel stores 4 scale bytes of consecutive blocks at once (any cols);
  // the tiled kernel stores the 4 of one row's 128 columns (cols % 128 == 0) or, with
  // 32x32 blocks, of 128 columns in one row of the scale grid (same condition)
  if (want_row && aligned(row_scales, 4) && (row_stream || s.cols % 128 == 0)) a.flags |= mx::kRowScaleDword;
  if (want_col && s.rows % 128 == 0 && aligned(col_scales, 4)) a.flags |= mx::kColScaleDword;
  if (want_row && want_col && !b2d && s.cols % 256 == 0 && aligned(row_scales, 8)) a.flags |= mx::kRowScaleQword;
  // Column-plane pitches that are multiples of 4 KiB: stagger the XCD strips so the
  // transposed stores in flight spread over the HBM channels. Measured on MI355X:
  // 16384-row 8-bit planes 4-7% faster; pitches like 14 KiB, tensors of fewer
  // than 64 tile rows and the 6-bit planes (ordinary stores) slightly slower.
  if (want_col && code_bits(fmt) != 6 && (s.rows * code_bits(fmt) / 8) % 4096 == 0 && g.tiles_r >= 64)
    a.flags |= mx::kStaggerStrips;
  const bool bf = x_dtype == MX_BF16;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const uint32_t nb = uint32_t(g.blocks);
  hipError_t e;
  if (sr) e = mx::launch_cast_sr(bf, int(fmt), int(mode), int(axis), b2d, a, nb, st);
  else if (b2d) e = mx::launch_cast_2d(bf, int(fmt), int(mode), int(axis), a, nb, st);
  else e = mx::launch_cast(bf, int(fmt), int(mode), int(axis), a, nb, st);
  return e == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}

int mx_copy_nt(const void* src, void* dst, int64_t bytes, void* stream) {
  if (src == nullptr || dst == nullptr) return MX_ERR_NULL;
  if (bytes <= 0 || bytes % 16 != 0) return MX_ERR_SHAPE;
  if (!aligned(src, 16) || !aligned(dst, 16)) return MX_ERR_ALIGN;
  if (overlap(range_of(src, bytes), range_of(dst, bytes))) return MX_ERR_ALIAS;
  if (mx::copy_blocks(bytes) > kMaxGrid) return MX_ERR_TOO_LARGE;
  const hipError_t e = mx::launch_copy_nt(src, dst, bytes, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}

int mx_dequantize(const void* codes, const uint8_t* scales, mx_fmt fmt, mx_shape s,
                  mx_dtype y_dtype, void* y, void* stream) {
  return mx_dequantize_ex(codes, scales, fmt, s, MX_BLOCK_1X32, y_dtype, y, stream);
}

int mx_dequantize_ex(const void* codes, const uint8_t* scales, mx_fmt fmt, mx_shape s, mx_block block,
                     mx_dtype y_dtype, void* y, void* stream) {
  if (!valid_fmt(fmt) || !valid_dtype(y_dtype) || !valid_block(block)) return MX_ERR_ENUM;
  if (codes == nullptr || scales == nullptr || y == nullptr) return MX_ERR_NULL;
  const bool b2d = block == MX_BLOCK_32X32;
  const int64_t n = elements(s);
  if (n < 0 || s.cols % kBlock != 0 || (b2d && s.rows % kBlock != 0)) return MX_ERR_SHAPE;
  if (!aligned(codes, dequant_code_align(fmt)) || !aligned(y, 16)) return MX_ERR_ALIGN;
  const Range rc = range_of(codes, n / 8 * code_bits(fmt));
  const Range rsc = range_of(scales, n / (b2d ? kBlock * kBlock : kBlock));
  const Range ry = range_of(y, n * (y_dtype == MX_BF16 ? 2 : 4));
  if (overlap(ry, rc) || overlap(ry, rsc)) return MX_ERR_ALIAS;
  if ((n / 16 + 255) / 256 > kMaxGrid) return MX_ERR_TOO_LARGE;
  const hipError_t e = mx::launch_dequant(int(fmt), y_dtype == MX_BF16, static_cast<const uint8_t*>(codes),
                                          scales, y, n, b2d ? s.cols : 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}

int mx_quantize_nvfp4(const void* x, mx_dtype x_dtype, mx_shape s, mx_axis axis, float* global_scale,
                      int global_given, void* row_codes, uint8_t* row_scales, void* col_codes,
                      uint8_t* col_scales, void* stream) {
  constexpr int64_t kNv = 16;
  if (!valid_dtype(x_dtype) || !valid_axis(axis) || (global_given != 0 && global_given != 1)) return MX_ERR_ENUM;
  const bool want_row = (axis & MX_AXIS_ROW) != 0;
  const bool want_col = (axis & MX_AXIS_COL) != 0;
  if (x == nullptr || global_scale == nullptr) return MX_ERR_NULL;
  if (want_row != (row_codes != nullptr) || want_row != (row_scales != nullptr)) return MX_ERR_NULL;
  if (want_col != (col_codes != nullptr) || want_col != (col_scales != nullptr)) return MX_ERR_NULL;
  const int64_t n = elements(s);
  if (n < 0 || s.cols % kNv != 0 || (want_col && s.rows % kNv != 0)) return MX_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(global_scale, 4) || (want_row && !aligned(row_codes, 16)) ||
      (want_col && !aligned(col_codes, 16)))
    return MX_ERR_ALIGN;
  Range rs[6];
  int nr = 0;
  rs[nr++] = range_of(x, n * (x_dtype == MX_BF16 ? 2 : 4));
  rs[nr++] = range_of(global_scale, s.batch * 4);
  if (want_row) { rs[nr++] = range_of(row_codes, n / 2); rs[nr++] = range_of(row_scales, n / kNv); }
  if (want_col) { rs[nr++] = range_of(col_codes, n / 2); rs[nr++] = range_of(col_scales, n / kNv); }
  for (int i = 0; i < nr; ++i)
    for (int j = i + 1; j < nr; ++j)
      if (overlap(rs[i], rs[j])) return MX_ERR_ALIAS;
  const mx::CastGrid g = mx::cast_grid(s.batch, s.rows, s.cols, false);
  if (g.blocks > kMaxGrid || s.batch > 65535) return MX_ERR_TOO_LARGE;
  if (s.cols >= (INT64_C(1) << 22) || (want_col && s.rows >= (INT64_C(1) << 23))) return MX_ERR_TOO_LARGE;

  mx::NvArgs a;
  a.x = x;
  a.row_codes = row_codes;
  a.row_scales = row_scales;
  a.col_codes = col_codes;
  a.col_scales = col_scales;
  a.global_scale = global_scale;
  a.rows = s.rows;
  a.cols = s.cols;
  a.tiles_r = uint32_t(g.tiles_r);
  a.tiles_c = uint32_t(g.tiles_c);
  a.flags = 0;
  if (want_row && s.cols % 64 == 0 && aligned(row_scales, 4)) a.flags |= mx::kRowScaleDword;
  if (want_col && s.rows % 64 == 0 && aligned(col_scales, 4)) a.flags |= mx::kColScaleDword;
  if (want_row && want_col && s.cols % 256 == 0 && aligned(row_scales, 16)) a.flags |= mx::kNvRowScaleWords;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf = x_dtype == MX_BF16;
  if (!global_given) {
    const hipError_t e = mx::launch_nvfp4_global(bf, x, s.batch, s.rows * s.cols, global_scale, st);
    if (e != hipSuccess) return MX_ERR_LAUNCH;
    a.flags |= mx::kNvMarkedAmax;
  }
  const hipError_t e = mx::launch_nvfp4_cast(bf, int(axis), a, uint32_t(g.blocks), st);
  return e == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}

int mx_dequantize_nvfp4(const void* codes, const uint8_t* scales, const float* global_scale, mx_shape s,
                        mx_dtype y_dtype, void* y, void* stream) {
  constexpr int64_t kNv = 16;
  if (!valid_dtype(y_dtype)) return MX_ERR_ENUM;
  if (codes == nullptr || scales == nullptr || global_scale == nullptr || y == nullptr) return MX_ERR_NULL;
  const int64_t n = elements(s);
  if (n < 0 || s.cols % kNv != 0) return MX_ERR_SHAPE;
  if (!aligned(codes, 8) || !aligned(y, 16) || !aligned(global_scale, 4)) return MX_ERR_ALIGN;
  const Range ry = range_of(y, n * (y_dtype == MX_BF16 ? 2 : 4));
  if (overlap(ry, range_of(codes, n / 2)) || overlap(ry, range_of(scales, n / kNv)) ||
      overlap(ry, range_of(global_scale, s.batch * 4)))
    return MX_ERR_ALIAS;
  if ((n / kNv + 255) / 256 > kMaxGrid) return MX_ERR_TOO_LARGE;
  const hipError_t e = mx::launch_nvfp4_dequant(y_dtype == MX_BF16, static_cast<const uint8_t*>(codes), scales,
                                                global_scale, y, n / kNv, s.rows * s.cols / kNv,
                                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}

// Shared by the two FP8-block entry points: the source is an MXFP4 plane
// (codes, scales) or master weights x (cast to MXFP4 on the way, optionally
// written to fp4_codes / fp4_scales).
static int rq_launch(int src, int mode, const void* x, const void* codes, const uint8_t* scales, uint8_t* fp4_codes,
                     uint8_t* fp4_scales, mx_shape s, mx_axis axis, uint8_t* fp8, float* block_scale,
                     uint8_t* fp8_t, float* block_scale_t, uint8_t* spread, void* stream) {
  const bool want_row = (axis & MX_AXIS_ROW) != 0;
  const bool want_col = (axis & MX_AXIS_COL) != 0;
  const bool from_mx = src == mx::kFromMx;
  const int64_t xes = src == mx::kFromF32 ? 4 : 2;
  if (from_mx ? (codes == nullptr || scales == nullptr) : x == nullptr) return MX_ERR_NULL;
  if ((fp4_codes != nullptr) != (fp4_scales != nullptr)) return MX_ERR_NULL;
  if (want_row != (fp8 != nullptr) || want_row != (block_scale != nullptr)) return MX_ERR_NULL;
  if (want_col != (fp8_t != nullptr) || want_col != (block_scale_t != nullptr)) return MX_ERR_NULL;
  const int64_t n = elements(s);
  if (n < 0 || s.cols % kBlock != 0 || (want_col && s.rows % 16 != 0)) return MX_ERR_SHAPE;
  if ((from_mx && !aligned(codes, 16)) || (!from_mx && !aligned(x, 16)) ||
      (fp4_codes != nullptr && !aligned(fp4_codes, 8)) ||
      (want_row && (!aligned(fp8, 16) || !aligned(block_scale, 4))) ||
      (want_col && (!aligned(fp8_t, 16) || !aligned(block_scale_t, 4))))
    return MX_ERR_ALIGN;
  const int64_t nbr = (s.rows + 127) / 128, nbc = (s.cols + 127) / 128;
  const int64_t nblk = s.batch * nbr * nbc;
  Range rs[8];
  int nr = 0;
  if (from_mx) {
    rs[nr++] = range_of(codes, n / 2);
    rs[nr++] = range_of(scales, n / kBlock);
  } else {
    rs[nr++] = range_of(x, n * xes);
    if (fp4_codes != nullptr) { rs[nr++] = range_of(fp4_codes, n / 2); rs[nr++] = range_of(fp4_scales, n / kBlock); }
  }
  if (want_row) { rs[nr++] = range_of(fp8, n); rs[nr++] = range_of(block_scale, nblk * 4); }
  if (want_col) { rs[nr++] = range_of(fp8_t, n); rs[nr++] = range_of(block_scale_t, nblk * 4); }
  if (spread != nullptr) rs[nr++] = range_of(spread, nblk);
  for (int i = 0; i < nr; ++i)
    for (int j = i + 1; j < nr; ++j)
      if (overlap(rs[i], rs[j])) return MX_ERR_ALIAS;
  if (s.cols >= (INT64_C(1) << 22) || (want_col && s.rows >= (INT64_C(1) << 23))) return MX_ERR_TOO_LARGE;
  const int64_t tiles_r = nbr, tiles_c = (s.cols + 255) / 256;
  const int64_t blocks = s.batch * tiles_r * tiles_c;
  if (blocks > UINT32_MAX / 2) return MX_ERR_TOO_LARGE;

  mx::RqArgs a;
  a.codes = static_cast<const uint8_t*>(codes);
  a.scales = scales;
  a.x = x;
  a.out_codes = fp4_codes;
  a.out_scales = fp4_scales;
  a.fp8 = fp8;
  a.block_scale = block_scale;
  a.fp8_t = fp8_t;
  a.block_scale_t = block_scale_t;
  a.spread = spread;
  a.rows = s.rows;
  a.cols = s.cols;
  a.tiles_r = uint32_t(tiles_r);
  a.tiles_c = uint32_t(tiles_c);
  a.total_tiles = uint32_t(blocks);
  a.flags = 0;
  // only with both copies: measured 2.2% faster there, but 2-3.5% slower for a
  // single copy
  if (src == mx::kFromMx && want_row && want_col && s.cols % 256 == 0 && aligned(scales, 4))
    a.flags |= mx::kRqScaleWords;
  // tile rows owned by one XCD each (the scale plane's lines then reach one L2):
  // measured 30.64 -> 30.34 us for 14336x4096 with both copies
  if (src == mx::kFromMx && (s.batch * tiles_r) % 8 == 0) a.flags |= mx::kRqXcdRows;
  const hipError_t e = mx::launch_requant(src, mode, int(axis), a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}

int mx_requant_fp4_fp8(const void* codes, const uint8_t* scales, mx_shape s, mx_axis axis, uint8_t* fp8,
                       float* block_scale, uint8_t* fp8_t, float* block_scale_t, uint8_t* spread, void* stream) {
  if (!valid_axis(axis)) return MX_ERR_ENUM;
  return rq_launch(mx::kFromMx, mx::kFloor, nullptr, codes, scales, nullptr, nullptr, s, axis, fp8, block_scale,
                   fp8_t, block_scale_t, spread, stream);
}

int mx_quantize_fp4_fp8(const void* x, mx_dtype x_dtype, mx_shape s, mx_scale_mode scale_mode, mx_axis axis,
                        void* fp4_codes, uint8_t* fp4_scales, uint8_t* fp8, float* block_scale, uint8_t* fp8_t,
                        float* block_scale_t, uint8_t* spread, void* stream) {
  if (!valid_dtype(x_dtype) || !valid_mode(scale_mode) || !valid_axis(axis)) return MX_ERR_ENUM;
  return rq_launch(x_dtype == MX_BF16 ? mx::kFromBf16 : mx::kFromF32,
                   scale_mode == MX_SCALE_ROUNDUP ? mx::kRoundUp : mx::kFloor, x, nullptr, nullptr,
                   static_cast<uint8_t*>(fp4_codes), fp4_scales, s, axis, fp8, block_scale, fp8_t, block_scale_t,
                   spread, stream);
}

}  // extern "C"
