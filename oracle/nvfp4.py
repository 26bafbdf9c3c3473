"""NVFP4: E2M1 elements, 16-element blocks with a UE4M3 scale, and an FP32
per-tensor global scale. TEST INFRASTRUCTURE, like the rest of ``oracle/``.

What the pages fix ([Q] "MXFP4 と NVFP4 は何が違うのか調べてみた", §3 and the §4
table): the elements are E2M1, exactly as in MXFP4; a block is 16 elements;
its scale is an unsigned E4M3 (UE4M3, largest value 448); a second, FP32 scale
per tensor brings the tensor's range in first, and is the tensor's largest
magnitude divided by 6 * 448; a 16-element block takes 16 * 4 + 8 = 72 bits
(4.5 bits per element); decoding multiplies by the FP8 block scale and the FP32
global scale. §7 warns that the block scale is unsigned.

The pages state what each scale is, not the arithmetic that produces the
codes (§7 counts the order of applying the two scales among the points an
implementation still has to get right). The plainest reading, taken here, is
the exact one:
every code is the round-to-nearest-even of an exact real quotient, and only the
two values the format itself stores in FP32 are rounded to FP32.

  * A = largest |x| over the tensor's finite elements (one tensor = one batch
    slice); g = the FP32 value nearest to A / 2688 (the stored global scale).
  * Block scale code: the UE4M3 value nearest to the exact quotient
    amax_b / (6 * g), ties to the even code, saturating at 448, sign bit 0.
  * Element code: the E2M1 value nearest to the exact quotient x / (s_b * g),
    s_b the decoded block scale, ties to the even code, saturating at 6; the
    sign bit is the sign of x (including -0).
  * Decoding: y = FP32 of the exact product e2m1 * s_b * g (one rounding;
    e2m1 * s_b is exact in FP32, so this equals fp32(fp32(e2m1 * s_b) * g),
    the FP8-then-FP32 multiply of the §4 table). BF16 output is that FP32
    value rounded to nearest-even. A NaN block scale decodes to NaN.

Readings where the pages give nothing (the quotient has no value):
  * a block whose scale code is 0 (an all-zero block, or a block whose amax is
    below half of UE4M3's smallest step relative to 6 * g) stores codes 0;
  * a g that is not a finite positive number (an all-zero tensor gives g = 0;
    a caller may pass any g) makes every block store scale 0 and codes 0;
  * a block holding NaN or +-Inf gets the UE4M3 NaN code 0x7F and element
    codes 0; A ignores non-finite elements.
  * Layout: codes as MXFP4 (two per byte, element 2k in the low nibble), block
    scales [B][R][C/16] (column copy [B][C][R/16]), global scales [B] FP32;
    the column copy is the same cast of X^T with the same global scale.

Exactness. Both roundings compare a numerator with (grid midpoint) x (divisor),
never dividing. Each such product is exact in float64: a UE4M3 midpoint has at
most 5 significant bits, 6 has 2 and an FP32 g 24 (31 bits in all); an E2M1
midpoint has at most 3 and s_b at most 4 (31 bits with g). The numerators are
FP32 or BF16 values, exact in float64, so every comparison is exact.
"""
from __future__ import annotations

import numpy as np

from .mx_oracle import E2M1, E4M3, ROW, COL, positive_grid, pack_e2m1, unpack_e2m1, value_table, widen, \
    f32_bits, bf16_bits

__all__ = ["NV_BLOCK", "nvfp4_global_scale", "nvfp4_quantize", "nvfp4_dequantize", "ue4m3_encode",
           "nearest_code_of_quotient"]

NV_BLOCK = 16          # [Q] §3 table: 16 elements per block
E2M1_MAX = 6.0         # [Q] §3: 6 is E2M1's largest value
UE4M3_MAX = 448.0      # [Q] §3: UE4M3 (FP8) tops out at 448
UE4M3_NAN = 0x7F


def _f32(v):
    return np.asarray(v, dtype=np.float32)


def nearest_code_of_quotient(num: np.ndarray, den: np.ndarray, fmt) -> np.ndarray:
    """Magnitude code of the value of fmt nearest to num / den, exactly.

    num >= 0 and den > 0 are float64 arrays (broadcast together) such that
    every product (midpoint of two neighbouring grid values) * den is exact in
    float64. The quotient is compared with the midpoints between neighbouring
    values of fmt's non-negative grid; at a midpoint the neighbour with the
    even code wins ([Q] §2: round to nearest, ties to even); beyond the
    largest value the largest value is taken ([Q] §4: clip).
    """
    codes, vals = positive_grid(fmt)
    mids = (vals[:-1] + vals[1:]) / 2                   # exact: a midpoint needs one bit more than its neighbours
    num, den = np.broadcast_arrays(np.asarray(num, np.float64), np.asarray(den, np.float64))
    num, den = num.reshape(-1), den.reshape(-1)
    out = np.empty(num.shape, np.int64)
    step = max(1, (1 << 22) // len(mids))               # bounds the threshold matrix to ~32 MB
    for i0 in range(0, num.size, step):
        n = num[i0:i0 + step, None]
        thr = mids[None, :] * den[i0:i0 + step, None]   # exact products (see the module note)
        idx = (n > thr).sum(axis=1)                     # midpoints strictly below num / den
        # a quotient exactly at midpoint idx goes up when the upper neighbour's code is even
        at = np.take_along_axis(n == thr, np.minimum(idx, len(mids) - 1)[:, None], axis=1)[:, 0] & (idx < len(mids))
        up = at & (codes[np.minimum(idx + 1, len(codes) - 1)] % 2 == 0)
        out[i0:i0 + step] = codes[idx + up.astype(np.int64)]
    return out


def nvfp4_global_scale(x64: np.ndarray) -> np.ndarray:
    """FP32 global scale per batch slice: the FP32 value nearest to A / (6 * 448),
    A over finite elements (IEEE float32 division rounds the exact quotient once)."""
    b = x64.shape[0]
    a = np.abs(np.where(np.isfinite(x64), x64, 0.0)).reshape(b, -1).max(axis=1)
    return _f32(a) / np.float32(E2M1_MAX * UE4M3_MAX)


def ue4m3_encode(amax: np.ndarray, g: np.ndarray) -> np.ndarray:
    """UE4M3 code nearest to amax / (6 * g) (amax >= 0 float64, g > 0 FP32), RNE, saturating at 448."""
    amax = np.asarray(amax, np.float64)
    den = np.float64(E2M1_MAX) * np.asarray(g, np.float64)      # exact: 2 + 24 bits
    return nearest_code_of_quotient(amax, den, E4M3).reshape(np.broadcast(amax, den).shape).astype(np.uint8)


def _quant_plane(x64: np.ndarray, g: np.ndarray):
    b, r, c = x64.shape
    blocks = x64.reshape(b, r, c // NV_BLOCK, NV_BLOCK)
    finite = np.isfinite(blocks)
    special = ~finite.all(axis=3)
    clean = np.where(finite, blocks, 0.0)
    amax = np.abs(clean).max(axis=3)                            # exact: inputs are FP32 or BF16
    g64 = np.asarray(g, np.float64).reshape(b, 1, 1)
    g_ok = np.isfinite(g64) & (g64 > 0)
    scode = ue4m3_encode(amax, np.where(g_ok, g64, 1.0) * np.ones_like(amax))
    scode = np.where(g_ok, scode, 0).astype(np.uint8)
    sval = value_table(E4M3)[scode.astype(np.int64)]
    den = (sval * np.where(g_ok, g64, 1.0))[..., None]          # s_b * g: exact in float64 (28 bits)
    zero = (scode == 0)[..., None] | special[..., None]
    mag = nearest_code_of_quotient(np.abs(clean), np.where(zero, 1.0, den) * np.ones_like(clean), E2M1)
    mag = mag.reshape(clean.shape)
    codes = mag | (np.signbit(clean).astype(np.int64) << 3)
    codes = np.where(zero, 0, codes).astype(np.uint8)
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
    """codes [B][N][M/2], scales [B][N][M/16], global_scale [B] -> FP32 / BF16 bits.

    y = e2m1 * s_b * g, formed exactly in float64 (at most 6 + 24 significant
    bits) and rounded once to FP32; BF16 output rounds that FP32 value."""
    c = unpack_e2m1(codes)
    b = c.shape[0]
    ev = value_table(E2M1)[c]
    sv = value_table(E4M3)[np.asarray(scales, dtype=np.int64)]
    sv = np.repeat(sv, NV_BLOCK, axis=-1)
    g = np.asarray(global_scale, np.float32).astype(np.float64).reshape((b,) + (1,) * (c.ndim - 1))
    nan = np.repeat(np.asarray(scales) == UE4M3_NAN, NV_BLOCK, axis=-1)
    with np.errstate(invalid="ignore"):
        y = np.where(nan, np.nan, ev * sv * g)
    bits32 = f32_bits(y)
    if out_dtype == "f32":
        return bits32
    if out_dtype == "bf16":
        y32 = bits32.view(np.float32).astype(np.float64)
        return bf16_bits(y32)
    raise ValueError(f"unknown output dtype {out_dtype!r}")
