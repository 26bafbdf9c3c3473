"""NVFP4: E2M1 elements, 16-element blocks with a UE4M3 scale, and an FP32
per-tensor global scale. TEST INFRASTRUCTURE, like the rest of ``oracle/``.

What the pages fix ([Q] "MXFP4 と NVFP4 は何が違うのか調べてみた", §3 and the §4
table): the elements are E2M1, exactly as in MXFP4; a block is 16 elements;
its scale is an unsigned E4M3 (UE4M3, largest value 448); a second, FP32 scale
per tensor brings the tensor's range in first, and is the tensor's largest
magnitude divided by 6 * 448; a 16-element block takes 16 * 4 + 8 = 72 bits
(4.5 bits per element); decoding multiplies by the FP8 block scale and the FP32
global scale. §7 warns that the block scale is unsigned.

The pages leave the arithmetic order open. Because floating point decides the
integer codes here, the readings below fix every step in FP32 (IEEE, round to
nearest-even), the precision the format itself names; this module performs
those steps with numpy float32 operations, one at a time:

  * A = largest |x| over the tensor's finite elements (one tensor = one batch
    slice); g = fp32(A / 2688) is the global (decode) scale.
  * Block scale: t = fp32(fp32(amax_b / 6) / g), encoded as E4M3 with
    round-to-nearest-even, saturating at 448, sign bit 0 (UE4M3).
  * Elements: q = fp32(x * r_b) with r_b = fp32(1 / fp32(s_b * g)) and s_b the
    decoded block scale (the §4 table applies NVFP4's scales by multiplication),
    encoded as E2M1 with round-to-nearest-even and saturation at 6.
  * A block whose scale code is 0 (all-zero blocks, and blocks too small for
    UE4M3 relative to g), whose r_b is not finite (fp32(s_b * g) is 0 or below
    2^-128), and every block of a tensor with g == 0, store codes 0.
  * A block holding NaN or +-Inf gets the UE4M3 NaN code 0x7F and element codes 0;
    A ignores non-finite elements.
  * Decoding: y = fp32(fp32(e2m1 * ue4m3) * g) (the first product is exact);
    BF16 output is that FP32 value rounded to nearest-even. A NaN block scale
    decodes to NaN.
  * Layout: codes as MXFP4 (two per byte, element 2k in the low nibble), block
    scales [B][R][C/16] (column copy [B][C][R/16]), global scales [B] FP32;
    the column copy is the same cast of X^T with the same global scale.
"""
from __future__ import annotations

import numpy as np

from .mx_oracle import E2M1, E4M3, ROW, COL, encode_elements, pack_e2m1, unpack_e2m1, value_table, widen, \
    bf16_bits

__all__ = ["NV_BLOCK", "nvfp4_global_scale", "nvfp4_quantize", "nvfp4_dequantize", "ue4m3_encode"]

NV_BLOCK = 16          # [Q] §3 table: 16 elements per block
E2M1_MAX = 6.0         # [Q] §3: 6 is E2M1's largest value
UE4M3_MAX = 448.0      # [Q] §3: UE4M3 (FP8) tops out at 448
UE4M3_NAN = 0x7F


def _f32(v):
    return np.asarray(v, dtype=np.float32)


def nvfp4_global_scale(x64: np.ndarray) -> np.ndarray:
    """FP32 global scale per batch slice: fp32(A / (6 * 448)), A over finite elements."""
    b = x64.shape[0]
    a = np.abs(np.where(np.isfinite(x64), x64, 0.0)).reshape(b, -1).max(axis=1)
    return _f32(a) / np.float32(E2M1_MAX * UE4M3_MAX)          # FP32 division, RNE


def ue4m3_encode(t: np.ndarray) -> np.ndarray:
    """Non-negative FP32 values -> E4M3 codes (sign bit 0), RNE, saturating at 448."""
    t = np.asarray(t, dtype=np.float64)
    return encode_elements(np.minimum(t, UE4M3_MAX), E4M3)


def _quant_plane(x64: np.ndarray, g: np.ndarray):
    b, r, c = x64.shape
    blocks = x64.reshape(b, r, c // NV_BLOCK, NV_BLOCK)
    finite = np.isfinite(blocks)
    special = ~finite.all(axis=3)
    clean = np.where(finite, blocks, 0.0)
    amax = _f32(np.abs(clean).max(axis=3))                      # exact: inputs are FP32 or BF16
    gg = g.reshape(b, 1, 1)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        t = (amax / np.float32(E2M1_MAX)) / gg                  # two FP32 divisions
    t = np.where(gg == 0, np.float32(0), t)
    scode = ue4m3_encode(t)
    sval = _f32(value_table(E4M3)[scode])
    den = sval * gg                                             # FP32 product
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        rb = np.float32(1) / den                                # FP32 division
        q = _f32(clean) * rb[..., None]                         # FP32 product
    zero = ((scode == 0) | ~np.isfinite(rb))[..., None]       # r_b overflows for a tiny s_b * g
    q = np.where(zero, np.float32(0), q)
    codes = encode_elements(q.astype(np.float64), E2M1)
    codes = np.where(zero, 0, codes).astype(np.uint8)
    codes = np.where(special[..., None], 0, codes).astype(np.uint8)
    scode = np.where(special, UE4M3_NAN, scode).astype(np.uint8)
    return pack_e2m1(codes.reshape(b, r, c)), scode


def nvfp4_quantize(x: np.ndarray, in_dtype: str, axis: int, global_scale: np.ndarray | None = None) -> dict:
    """NVFP4 cast of a [B][R][C] (or [R][C]) tensor.

    Returns global_scale [B] (float32) and row_codes/row_scales and/or
    col_codes/col_scales. A caller-given global_scale is used as is.
    """
    x64 = widen(x, in_dtype)
    if x64.ndim == 2:
        x64 = x64[None]
    g = nvfp4_global_scale(x64) if global_scale is None else _f32(global_scale).reshape(-1)
    out = {"global_scale": g}
    if axis & ROW:
        out["row_codes"], out["row_scales"] = _quant_plane(x64, g)
    if axis & COL:
        out["col_codes"], out["col_scales"] = _quant_plane(np.ascontiguousarray(x64.transpose(0, 2, 1)), g)
    return out


def nvfp4_dequantize(codes: np.ndarray, scales: np.ndarray, global_scale: np.ndarray, out_dtype: str):
    """codes [B][N][M/2], scales [B][N][M/16], global_scale [B] -> FP32 / BF16 bits."""
    c = unpack_e2m1(codes)
    b = c.shape[0]
    ev = _f32(value_table(E2M1)[c])
    sv = _f32(value_table(E4M3)[np.asarray(scales, dtype=np.int64)])
    sv = np.repeat(sv, NV_BLOCK, axis=-1)
    g = _f32(global_scale).reshape((b,) + (1,) * (c.ndim - 1))
    y = (ev * sv) * g                                           # FP32: exact product, then one rounding
    nan = np.repeat(np.asarray(scales) == UE4M3_NAN, NV_BLOCK, axis=-1)
    y = np.where(nan, np.float32(np.nan), y)
    bits = y.view(np.uint32).copy()
    bits[np.isnan(y)] = 0x7FC00000
    if out_dtype == "f32":
        return bits
    if out_dtype == "bf16":
        return bf16_bits(y.astype(np.float64))
    raise ValueError(f"unknown output dtype {out_dtype!r}")
