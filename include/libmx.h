/* libmx: OCP Microscaling (MX) block quantization on AMD Instinct MI355X (gfx950).
 *
 * The operation ("MXFP4 と NVFP4 は何が違うのか調べてみた", §2 MX family table and
 * E8M0 paragraph, §4 "精度の差はどこから出るか"):
 *   - a tensor is cut into blocks of 32 consecutive elements;
 *   - each block gets one shared E8M0 scale: a power of two 2^e stored as the
 *     byte e + 127 (codes 0..254 <-> 2^-127..2^127; 0xFF is NaN, no Inf);
 *   - each element is stored as x / 2^e in the element format, MXFP8
 *     (E4M3 or E5M2, 8.25 bits per element with the scale) or MXFP4 (E2M1,
 *     two codes per byte, 4.25 bits per element), rounded to nearest-even
 *     and clipped at the format's largest value;
 *   - dequantization multiplies a code's value by its block's scale, an
 *     exponent add with no rounding error (§7); a NaN scale makes the
 *     whole block NaN (§2).
 * The quantized data and the scales live in separate planes, one scale byte
 * per 32 elements (§9, the Metal UE8M0 scale plane with 32x1 blocks).
 *
 * Conventions shared by every call:
 *   - Tensors are dense, row-major [batch][rows][cols]; cols is the
 *     contiguous axis.
 *   - Every data pointer is a device pointer allocated and owned by the
 *     caller; libmx never allocates, frees or keeps memory, and keeps no
 *     global state.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously; nothing synchronizes inside libmx.
 *     Device-side faults surface at the caller's next synchronization.
 *   - Return value: MX_OK (0) or a negative MX_ERR_* code. Argument errors are
 *     reported synchronously, before any HIP call. No exception crosses the ABI.
 */
#ifndef LIBMX_H
#define LIBMX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element formats. E4M3: bias 7, max 448, no Inf, NaN = S.1111.111.
 * E5M2: bias 15, max 57344, IEEE Inf/NaN. E2M1: bias 1, values
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives, no Inf/NaN.
 * The other rows of the same article's §2 family table (MXFP6, 6.25 bits per
 * element; MXINT8, 8.25), read as the OCP elements:
 * E2M3: sign in bit 5, 2 exponent bits (bias 1), 3 mantissa bits, max 7.5;
 * E3M2: sign in bit 5, 3 exponent bits (bias 3), 2 mantissa bits, max 28;
 *       both with subnormals and without Inf/NaN; 4 codes per 3 bytes, the
 *       codes forming a little-endian bit stream (element i in bits 6i..6i+5);
 * INT8: two's-complement k meaning k/64 (max 127/64, emax 0), rounded to
 *       nearest-even and clipped to +-127 (-128 is never produced). */
typedef enum {
  MX_E4M3 = 0, MX_E5M2 = 1, MX_E2M1 = 2, MX_E2M3 = 3, MX_E3M2 = 4, MX_INT8 = 5
} mx_fmt;

/* Shared-exponent rules (same article, §4 and the rounding paragraph of §2):
 * MX_SCALE_FLOOR   e = floor(log2(amax)) - emax (OCP example rule; the scaled
 *                  block max lands in [2^emax, 2^(emax+1)), the excess clips);
 * MX_SCALE_ROUNDUP the smallest e with amax <= max * 2^e (no clipping; the
 *                  scaled block max lands in (max/2, max]).
 * emax = floor(log2(max)): 8 (E4M3), 15 (E5M2), 2 (E2M1, E2M3), 4 (E3M2),
 * 0 (INT8). e is clamped to [-127, 127]; an all-zero block gets code 0x00. A
 * block holding a NaN or an Inf gets scale 0xFF and element codes 0x7F (FP8)
 * or 0x0 (formats with no NaN code). */
typedef enum { MX_SCALE_FLOOR = 0, MX_SCALE_ROUNDUP = 1 } mx_scale_mode;

typedef enum { MX_F32 = 0, MX_BF16 = 1 } mx_dtype;

/* Bitmask. ROW: blocks of 32 along cols. COL: blocks of 32 rows of one column,
 * stored transposed (the column copy is the row-wise quantization of X^T). */
typedef enum { MX_AXIS_ROW = 1, MX_AXIS_COL = 2, MX_AXIS_BOTH = 3 } mx_axis;

typedef struct {
  int64_t batch, rows, cols;
} mx_shape;

/* Rounding of the elements (same article: §2 requires round-to-nearest-even for
 * the FP4 conversion; §4's 4-bit pretraining recipe rounds gradients
 * stochastically, and §8 lists stochastic rounding among the P3109 modes).
 * MX_ROUND_STOCHASTIC: a scaled value s with |s| < max goes to the grid value
 *   above |s| when the fraction f of |s| between its two neighbouring grid
 *   values exceeds u / 2^16, else to the one below; |s| >= max saturates; the
 *   sign is kept. u is 16 bits of Philox4x32-10 (Salmon et al., SC'11) keyed
 *   by the 64-bit seed (key word 0 = low half): element i of X's flat
 *   [batch][rows][cols] order uses the output block of counter
 *   (i >> 3, 0, 0) (the 64-bit i >> 3 in words 0-1), its word (i >> 1) & 3,
 *   low half for even i, high half for odd i. The row and column copies of an
 *   element use the same u. Scales are chosen as for nearest-even. */
typedef enum { MX_ROUND_NEAREST_EVEN = 0, MX_ROUND_STOCHASTIC = 1 } mx_rounding;

/* Block shape (same article §4: the recipe scales weights in two-dimensional
 * blocks). MX_BLOCK_32X32: one E8M0 scale per 32x32 tile of each batch slice,
 * chosen from the tile's largest magnitude by the same rules; the row copy's
 * scale plane is [batch][rows/32][cols/32] and the column copy (the same cast
 * of X^T) has codes [batch][cols][rows'] and scales [batch][cols/32][rows/32].
 * rows and cols must both be multiples of 32. */
typedef enum { MX_BLOCK_1X32 = 0, MX_BLOCK_32X32 = 1 } mx_block;

typedef struct {
  mx_rounding rounding;
  mx_block block;
  uint64_t seed;        /* used by MX_ROUND_STOCHASTIC only */
} mx_quant_opts;

#define MX_OK 0
#define MX_ERR_NULL (-1)        /* a required pointer is NULL, or an unused one is not */
#define MX_ERR_SHAPE (-2)       /* non-positive extent, or a blocked extent not a multiple of the block */
#define MX_ERR_ALIGN (-3)       /* a pointer without the alignment its call requires */
#define MX_ERR_ENUM (-4)        /* unknown fmt / mode / dtype / axis */
#define MX_ERR_ALIAS (-5)       /* input and an output overlap, or two outputs do */
#define MX_ERR_TOO_LARGE (-6)   /* beyond one launch: cols >= 2^22, rows >= 2^23 with
                                   column planes, or more than 2^31-1 tiles */
#define MX_ERR_LAUNCH (-7)      /* a kernel launch failed (the status hipLaunchKernel returned for it;
                                   an error left by an unrelated earlier call is not read or cleared) */

/* Bytes of the code planes and of the scale planes that mx_quantize writes for
 * a tensor of shape s, format fmt and the planes selected by axis (1x32
 * blocks): each plane holds batch*rows*cols*bits/8 code bytes (bits 8, 6 or 4)
 * and batch*rows*cols/32 scale bytes, and *code_bytes / *scale_bytes receive
 * the totals over the selected planes (twice one plane for MX_AXIS_BOTH).
 * Per element and plane that is bits + 8/32: 4.25 bits for MXFP4 and 8.25 for
 * MXFP8 (same article, §2 family table; 6.25 for MXFP6, 8.25 for MXINT8).
 * Shape rules: extents >= 1; cols % 32 == 0 with MX_AXIS_ROW; rows % 32 == 0
 * with MX_AXIS_COL. Errors: MX_ERR_ENUM, MX_ERR_NULL, MX_ERR_SHAPE. Pure host
 * arithmetic; no HIP call. */
int mx_plane_bytes(mx_fmt fmt, mx_shape s, mx_axis axis, size_t* code_bytes, size_t* scale_bytes);

/* Quantize x ([batch][rows][cols], x_dtype) into the planes selected by axis.
 *   row_codes  [batch][rows][cols] bytes, E2M1: [batch][rows][cols/2] with
 *              element 2k in bits 3:0 and element 2k+1 in bits 7:4,
 *              E2M3/E3M2: [batch][rows][3*cols/4]
 *   row_scales [batch][rows][cols/32] E8M0 bytes
 *   col_codes  [batch][cols][rows] bytes, E2M1: [batch][cols][rows/2],
 *              E2M3/E3M2: [batch][cols][3*rows/4]
 *   col_scales [batch][cols][rows/32]
 * Pointers of an axis not in `axis` must be NULL; the others must be non-NULL.
 * Shape: batch, rows, cols >= 1; cols % 32 == 0 when MX_AXIS_ROW is set (the
 * row blocks); rows % 32 == 0 when MX_AXIS_COL is set (the column blocks).
 * A column-only cast blocks no run along cols, which then needs only rows of
 * whole 16-byte vectors: cols % 8 == 0 (BF16) or cols % 4 == 0 (FP32).
 * x, row_codes and col_codes must be 16-byte aligned. Inputs and outputs must
 * not overlap. */
int mx_quantize(const void* x, mx_dtype x_dtype, mx_shape s, mx_fmt fmt, mx_scale_mode mode,
                mx_axis axis, void* row_codes, uint8_t* row_scales, void* col_codes,
                uint8_t* col_scales, void* stream);

/* Dequantize one plane. s is the shape of the plane as stored, with blocks of
 * 32 along s.cols (a column plane is passed as [batch][cols][rows] and comes
 * out as X^T). codes: batch*rows*cols bytes (E2M1: half, E2M3/E3M2: three
 * quarters); scales: batch*rows*cols/32 bytes; y: batch*rows*cols elements of
 * y_dtype. FP32 output is exact; BF16 output is the exact value rounded to
 * nearest-even. NaN is written as 0x7FC00000 (FP32) / 0x7FC0 (BF16).
 * Shape: extents >= 1, cols % 32 == 0. y 16-byte aligned; codes 16-byte
 * aligned (E2M1 8-byte, E2M3/E3M2 4-byte). y must not overlap codes or scales. */
int mx_dequantize(const void* codes, const uint8_t* scales, mx_fmt fmt, mx_shape s,
                  mx_dtype y_dtype, void* y, void* stream);

/* mx_quantize with options; opts == NULL means nearest-even and 1x32 blocks,
 * which is exactly mx_quantize. With MX_BLOCK_32X32 the scale planes hold
 * batch*rows*cols/1024 bytes each (layout above) and rows % 32 == 0 and
 * cols % 32 == 0 for every axis; the code planes are as for mx_quantize. Errors as mx_quantize,
 * plus MX_ERR_ENUM for an unknown rounding or block. The result depends only on
 * the inputs, the options and the seed (not on the launch or the device). */
int mx_quantize_ex(const void* x, mx_dtype x_dtype, mx_shape s, mx_fmt fmt, mx_scale_mode mode,
                   mx_axis axis, const mx_quant_opts* opts, void* row_codes, uint8_t* row_scales,
                   void* col_codes, uint8_t* col_scales, void* stream);

/* mx_dequantize for either block shape. With MX_BLOCK_32X32, scales is the
 * [batch][rows/32][cols/32] grid of the plane as stored (a column plane passes
 * [batch][cols][rows] with its [batch][cols/32][rows/32] grid) and rows % 32
 * must be 0. MX_BLOCK_1X32 is exactly mx_dequantize. */
int mx_dequantize_ex(const void* codes, const uint8_t* scales, mx_fmt fmt, mx_shape s, mx_block block,
                     mx_dtype y_dtype, void* y, void* stream);

/* NVFP4 (same article, §3, the §4 table and §7): E2M1 elements (MXFP4's) in
 * blocks of 16, each with an unsigned E4M3 (UE4M3, at most 448, sign bit 0)
 * block scale, and one FP32 global scale per tensor (per batch slice) equal
 * to the slice's largest finite magnitude A over 6 * 448; 4.5 bits per
 * element. The codes are exact roundings of exact quotients:
 * g = fp32(A / 2688); the block code is the UE4M3 value nearest to
 * amax_b / (6 g) (ties to the even code, saturating at 448); each element
 * code is the E2M1 value nearest to x / (s_b g) (ties to even, saturating at
 * 6, sign of x). A block whose scale code is 0, and every block when g is
 * not a finite positive number, stores codes 0; a block holding NaN or Inf
 * stores scale 0x7F (UE4M3 NaN) and codes 0.
 *   global_scale  [batch] FP32, device memory: written (global_given == 0)
 *                 or read (global_given == 1, e.g. a scale kept from an
 *                 earlier step). When written, it holds intermediate values
 *                 (each slice's raw maximum with the sign bit set) until the
 *                 stream has run the whole call, and g afterwards.
 *   row_codes     [batch][rows][cols/2] (element 2k in bits 3:0)
 *   row_scales    [batch][rows][cols/16] UE4M3 bytes
 *   col_codes     [batch][cols][rows/2]  (the same cast of X^T)
 *   col_scales    [batch][cols][rows/16]
 * Shape: cols % 16 == 0, rows % 16 == 0 with MX_AXIS_COL, batch <= 65535.
 * x, row_codes and col_codes 16-byte aligned, global_scale 4-byte aligned.
 * Computing g reads x once more than the cast (one extra pass). */
int mx_quantize_nvfp4(const void* x, mx_dtype x_dtype, mx_shape s, mx_axis axis, float* global_scale,
                      int global_given, void* row_codes, uint8_t* row_scales, void* col_codes,
                      uint8_t* col_scales, void* stream);

/* NVFP4 dequantization of one plane ([batch][rows][cols] as stored, blocks of
 * 16 along cols): y = (e2m1 * ue4m3) * g in FP32 (the first product is exact),
 * BF16 output rounded to nearest-even from that FP32 value; a NaN block scale
 * gives the canonical NaN. codes 8-byte aligned, y 16-byte aligned. */
int mx_dequantize_nvfp4(const void* codes, const uint8_t* scales, const float* global_scale, mx_shape s,
                        mx_dtype y_dtype, void* y, void* stream);

/* FP4-in-FP8 nested requantization (same article, §6, DeepSeek-V4's nested
 * structure): an MXFP4 plane (E2M1 codes two per byte, one E8M0 scale per 32
 * elements along cols, as mx_quantize writes it) re-expressed as FP8 E4M3
 * with one FP32 scale per 128x128 block, which holds 512 of the 1x32
 * sub-blocks. A sub-block is active when one of its codes has a nonzero
 * magnitude and its scale is not 0xFF; kmax / kmin are the largest and
 * smallest scale codes of a block's active sub-blocks. The block scale is
 * S = 2^(kmax - 133) (1.0 for a block without active sub-blocks), so E2M1's 6
 * at kmax lands on 384; element e2m1 * 2^(k - 127) is stored as the E4M3 code
 * of its value / S, rounded to nearest-even, 0x7F in a NaN sub-block, zeros
 * keeping their sign. spread = kmax - kmin (0 with fewer than two active
 * sub-blocks) is the check the article asks for: spread <= 14 (a scale ratio
 * of at most 2^14) makes every value / S an E4M3 value, so the block converts
 * exactly; above that, the smallest sub-blocks can lose their 0.5 and 1.5.
 * Blocks at a ragged edge cover the rows and columns present.
 *   codes          [batch][rows][cols/2], 16-byte aligned; scales [batch][rows][cols/32]
 *   fp8            [batch][rows][cols] E4M3, 16-byte aligned  (MX_AXIS_ROW)
 *   block_scale    [batch][R'][C'] FP32, R' = ceil(rows/128), C' = ceil(cols/128)
 *   fp8_t          [batch][cols][rows]: the same codes transposed (MX_AXIS_COL;
 *                  the square blocks make the transposed weight need no new
 *                  quantization), 16-byte aligned, rows % 16 == 0
 *   block_scale_t  [batch][C'][R'] FP32 (the transposed grid)
 *   spread         [batch][R'][C'] bytes, or NULL
 * Shape: cols % 32 == 0. Pointers of an axis not requested must be NULL. */
int mx_requant_fp4_fp8(const void* codes, const uint8_t* scales, mx_shape s, mx_axis axis, uint8_t* fp8,
                       float* block_scale, uint8_t* fp8_t, float* block_scale_t, uint8_t* spread, void* stream);

/* The quantization-aware step of the same section in one pass: master weights
 * x (BF16 or FP32, [batch][rows][cols]) are cast to MXFP4 exactly as
 * mx_quantize does with fmt = MX_E2M1, scale rule scale_mode and
 * MX_AXIS_ROW, and that MXFP4 plane is re-expressed as FP8 exactly as
 * mx_requant_fp4_fp8 does; the result equals the two calls in sequence.
 *   fp4_codes / fp4_scales  the MXFP4 plane ([batch][rows][cols/2], 8-byte
 *                aligned; [batch][rows][cols/32]), both or neither (NULL: not stored)
 *   fp8, block_scale, fp8_t, block_scale_t, spread  as for mx_requant_fp4_fp8
 * x 16-byte aligned; cols % 32 == 0; rows % 16 == 0 with MX_AXIS_COL. */
int mx_quantize_fp4_fp8(const void* x, mx_dtype x_dtype, mx_shape s, mx_scale_mode scale_mode, mx_axis axis,
                        void* fp4_codes, uint8_t* fp4_scales, uint8_t* fp8, float* block_scale, uint8_t* fp8_t,
                        float* block_scale_t, uint8_t* spread, void* stream);

/* Measurement helper, not an MX operation: copies `bytes` from src to dst with
 * 16-byte non-temporal loads and stores, one chunk per thread. It moves the
 * same kind of read and write traffic as a cast with no arithmetic, which makes
 * it the bandwidth ceiling the casts are compared against. src and dst are
 * caller-owned device memory, 16-byte aligned, not overlapping;
 * bytes > 0 and bytes % 16 == 0. Enqueued on `stream`. Errors: MX_ERR_NULL,
 * MX_ERR_SHAPE (size), MX_ERR_ALIGN, MX_ERR_ALIAS, MX_ERR_TOO_LARGE,
 * MX_ERR_LAUNCH. */
int mx_copy_nt(const void* src, void* dst, int64_t bytes, void* stream);

/* Static text for an MX_* code; never NULL. */
const char* mx_strerror(int err);

/* Library version as major*10000 + minor*100 + patch. */
int mx_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBMX_H */
