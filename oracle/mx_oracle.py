"""MX block quantization: a plain, exact CPU oracle.

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module. It shares no
code with the HIP library (no headers, tables, helpers or constants), and
neither side imports the other.

Everything is computed in float64 with NumPy, where every step below is exact
(inputs are BF16 or FP32, which widen exactly; scales are powers of two).
The element encoder is a nearest-value search over each format's table of
representable values, which is deliberately a different algorithm from the bit
manipulation or conversion hardware a GPU path would use.

Sources, cited by tag:
  [Q]   "MXFP4 と NVFP4 は何が違うのか調べてみた" (qiita.com), by section.
  [OSS] news repost "OpenAI 在最新的开源模型 gpt-oss 上选用的 MXFP4 数据类型"
        (m.lxslee.cn), its "MXFP4" section with the four-value example.
  [R8]  summary of "Recipes for Pre-training LLMs with MXFP8" (aibr.jp), §3.
FP8 bit layouts (bias, subnormals, NaN and Inf codes) are not printed on the
pages; they follow the OCP 8-bit floating-point definitions that [Q] §2 and §8
refer to, and the tests pin them against torch's float8 types.
[Q] §2's family table also lists MXFP6 (E2M3 or E3M2, 6.25 bits per element)
and MXINT8 (INT8, 8.25 bits per element) with the same 32-element blocks and
E8M0 scale, but prints no bit layout for them; the readings below fill that in.

Readings taken where the pages are silent (each is listed in the design doc):
  * emax of a format is floor(log2(max finite)): 2 (E2M1), 8 (E4M3), 15 (E5M2).
  * FP8 elements use round-to-nearest-even like FP4.
  * Overflow saturates to +-max for every format.
  * A block holding any NaN or +-Inf gets scale 0xFF; its element codes are
    0x7F (FP8, a NaN code) or 0x0 (formats with no NaN code).
  * An all-zero block gets scale code 0x00 (2^-127); its codes are +-0.
  * Round-up scale rule = the smallest e with amax <= max * 2^e, exactly.
  * E2M1 packing: element 2k in bits 3:0, element 2k+1 in bits 7:4.
  * E2M3 / E3M2: sign, then 2 / 3 exponent bits with bias 2^(E-1) - 1 (1 / 3),
    then 3 / 2 mantissa bits, subnormals at exponent field 0, and no Inf or
    NaN (every code is a number, as in E2M1): maxima 7.5 and 28, emax 2 and 4.
  * 6-bit packing generalizes the E2M1 nibble order: codes form a little-endian
    bit stream, element i in stream bits 6i .. 6i+5, byte j holding stream
    bits 8j .. 8j+7 (4 codes in 3 bytes).
  * INT8 elements are two's-complement bytes read as k / 64 (the OCP MXINT8
    element, emax 0, largest value 127/64). Saturation is symmetric: the code
    -128 (-2.0) is never produced, so encoding keeps code(-x) = -code(x); -0
    encodes as 0. Formats with no NaN code fill a NaN/Inf block with code 0.
  * The column-wise copy is stored transposed: column-wise(X) = row-wise(X^T).
  * Dequantized values are rounded to the output type with RNE; NaN is written
    as the positive quiet NaN 0x7FC00000 (FP32) or 0x7FC0 (BF16).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = [
    "Fmt", "E4M3", "E5M2", "E2M1", "E2M3", "E3M2", "INT8", "FORMATS", "FLOOR", "ROUNDUP", "ROW", "COL", "BOTH",
    "BLOCK", "decode_code", "value_table", "max_finite", "emax_of", "positive_grid",
    "widen", "encode_elements", "shared_exponent", "quantize_blocks", "quantize",
    "pack_e2m1", "unpack_e2m1", "pack_fp6", "unpack_fp6", "pack_codes", "unpack_codes", "dequantize", "round_to_binary", "f32_bits",
    "bf16_bits", "plane_bytes",
]

BLOCK = 32            # [Q] §2, MXFP4 table: 32 elements share one scale; [OSS]: default 32
FLOOR, ROUNDUP = 0, 1  # [Q] §4 "精度の差はどこから出るか": the two scale conventions
ROW, COL, BOTH = 1, 2, 3
E8M0_BIAS = 127        # [Q] §2: E8M0, bias 127, codes 0..254 <-> 2^-127..2^127
E8M0_NAN = 0xFF        # [Q] §2: 0xFF is NaN, there is no Inf


@dataclass(frozen=True)
class Fmt:
    """A sign / exponent / mantissa element format, or a fixed-point integer one."""
    name: str
    ebits: int
    mbits: int
    bias: int
    ieee_specials: bool   # E5M2: all-ones exponent holds Inf (m=0) and NaN (m!=0)
    nan_all_ones: bool    # E4M3: only S.1111.111 is NaN, no Inf
    integer: bool = False  # two's-complement integer; bias = number of fraction bits

    @property
    def bits(self) -> int:
        return 1 + self.ebits + self.mbits

    @property
    def has_nan(self) -> bool:
        return self.ieee_specials or self.nan_all_ones


# [Q] §1: E2M1 = 1 sign, 2 exponent, 1 mantissa bit, no Inf and no NaN.
E2M1 = Fmt("e2m1", 2, 1, 1, False, False)
# [R8] §3: E4M3 = 4 exponent + 3 mantissa bits; [Q] §3: its max is 448 (this pins
# the variant without Inf whose only NaN is S.1111.111, bias 7).
E4M3 = Fmt("e4m3", 4, 3, 7, False, True)
# [Q] §2 MX family table lists E5M2 as the other MXFP8 element (bias 15, IEEE Inf/NaN).
E5M2 = Fmt("e5m2", 5, 2, 15, True, False)
# [Q] §2 MX family table: MXFP6 takes E2M3 or E3M2 elements (6.25 bits per element).
E2M3 = Fmt("e2m3", 2, 3, 1, False, False)
E3M2 = Fmt("e3m2", 3, 2, 3, False, False)
# [Q] §2 MX family table: MXINT8 (8.25 bits per element); read as k / 2^6.
INT8 = Fmt("int8", 0, 7, 6, False, False, integer=True)
FORMATS = {"e4m3": E4M3, "e5m2": E5M2, "e2m1": E2M1, "e2m3": E2M3, "e3m2": E3M2, "int8": INT8}


def decode_code(fmt: Fmt, code: int) -> float:
    """Value of one element code, from the bit definition of the format."""
    if fmt.integer:
        k = code - (1 << fmt.bits) if code >> (fmt.bits - 1) else code
        return k * 2.0 ** -fmt.bias
    sign = -1.0 if (code >> (fmt.bits - 1)) & 1 else 1.0
    exp = (code >> fmt.mbits) & ((1 << fmt.ebits) - 1)
    man = code & ((1 << fmt.mbits) - 1)
    all_ones = (1 << fmt.ebits) - 1
    if fmt.ieee_specials and exp == all_ones:
        return sign * float("inf") if man == 0 else float("nan")
    if fmt.nan_all_ones and exp == all_ones and man == (1 << fmt.mbits) - 1:
        return float("nan")
    if exp == 0:   # subnormal: 0.m * 2^(1 - bias)
        return sign * (man / (1 << fmt.mbits)) * 2.0 ** (1 - fmt.bias)
    return sign * (1.0 + man / (1 << fmt.mbits)) * 2.0 ** (exp - fmt.bias)


def value_table(fmt: Fmt) -> np.ndarray:
    """float64 value of every code 0 .. 2^bits - 1 (NaN / +-Inf where defined)."""
    return np.array([decode_code(fmt, c) for c in range(1 << fmt.bits)], dtype=np.float64)


def max_finite(fmt: Fmt) -> float:
    t = value_table(fmt)
    return float(np.max(t[np.isfinite(t)]))


def emax_of(fmt: Fmt) -> int:
    """Largest binade of the element format: floor(log2(max)). [Q] §4 gives 2 for E2M1."""
    return int(np.frexp(max_finite(fmt))[1]) - 1


def positive_grid(fmt: Fmt):
    """(codes, values) of the non-negative finite codes, sorted by value."""
    t = value_table(fmt)
    codes = np.arange(1 << (fmt.bits - 1))          # sign bit clear
    vals = t[codes]
    keep = np.isfinite(vals)
    codes, vals = codes[keep], vals[keep]
    order = np.argsort(vals, kind="stable")
    return codes[order].astype(np.int64), vals[order]


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 copy of BF16 bit patterns (uint16) or FP32 values."""
    if dtype == "bf16":
        u = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown input dtype {dtype!r}")


def encode_elements(s: np.ndarray, fmt: Fmt) -> np.ndarray:
    """Element codes of already-scaled finite values s (float64).

    [Q] §2 ("丸めについては"): conversion rounds to nearest, ties to even. The
    nearest representable value is found in the sorted table; at an exact
    midpoint the neighbour whose code is even wins. [Q] §4: values beyond the
    largest representable magnitude are clipped to it. The sign is copied from
    s, including the sign of zero; an integer format negates the magnitude
    code in two's complement instead (so -0 and +0 share code 0).
    """
    codes_pos, vals_pos = positive_grid(fmt)
    n = len(vals_pos)
    a = np.abs(s)
    idx = np.searchsorted(vals_pos, a, side="left")     # vals_pos[idx-1] < a <= vals_pos[idx]
    hi = np.minimum(idx, n - 1)
    lo = np.maximum(idx - 1, 0)
    d_lo = a - vals_pos[lo]
    d_hi = vals_pos[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes_pos[hi] % 2 == 0))
    mag = np.where(pick_hi, codes_pos[hi], codes_pos[lo])
    mag = np.where(a >= vals_pos[-1], codes_pos[-1], mag)  # saturate at +-max
    if fmt.integer:
        neg = np.signbit(s)
        return np.where(neg, (-mag) & ((1 << fmt.bits) - 1), mag).astype(np.uint8)
    sign = np.signbit(s).astype(np.int64) << (fmt.bits - 1)
    return (mag | sign).astype(np.uint8)


def shared_exponent(amax: np.ndarray, fmt: Fmt, mode: int) -> np.ndarray:
    """Unbiased shared exponent e of finite, non-negative block maxima.

    FLOOR ([Q] §4): e = floor(log2(amax)) - emax, so the scaled block max lands
    in [2^emax, 2^(emax+1)) and the part above max is clipped.
    ROUNDUP ([Q] §2 and §4): one step larger whenever the floor rule would clip,
    i.e. the smallest e with amax <= max * 2^e; the scaled max lands in
    (max/2, max].
    Both are clamped to the E8M0 range [-127, 127] ([Q] §2). An all-zero block
    takes e = -127.
    """
    amax = np.asarray(amax, dtype=np.float64)
    em = emax_of(fmt)
    vmax = max_finite(fmt)
    mant, ex = np.frexp(amax)                 # amax = mant * 2^ex, mant in [0.5, 1)
    big_e = ex.astype(np.int64) - 1           # floor(log2(amax)) for amax > 0
    e = big_e - em
    if mode == ROUNDUP:
        e = e + (amax > np.ldexp(vmax, big_e - em)).astype(np.int64)
    elif mode != FLOOR:
        raise ValueError(f"unknown scale mode {mode}")
    e = np.where(amax == 0, -E8M0_BIAS, e)
    return np.clip(e, -E8M0_BIAS, E8M0_BIAS).astype(np.int64)


def quantize_blocks(blocks: np.ndarray, fmt: Fmt, mode: int):
    """Quantize rows of 32 float64 values; returns (codes uint8 [n,32], scales uint8 [n]).

    [Q] §2: one E8M0 scale per block of 32; elements are stored as x / 2^e in the
    element format. A NaN scale makes all 32 elements NaN, so a block holding a
    NaN or an Inf (E8M0 has no Inf) gets scale 0xFF.
    """
    blocks = np.asarray(blocks, dtype=np.float64)
    assert blocks.ndim == 2 and blocks.shape[1] == BLOCK
    special = ~np.isfinite(blocks).all(axis=1)
    clean = np.where(special[:, None], 0.0, blocks)
    amax = np.max(np.abs(clean), axis=1) if len(clean) else np.zeros(0)
    e = shared_exponent(amax, fmt, mode)
    s = np.ldexp(clean, -e[:, None])              # exact: division by a power of two
    codes = encode_elements(s, fmt)
    codes[special] = 0x7F if fmt.has_nan else 0x0
    scales = (e + E8M0_BIAS).astype(np.uint8)
    scales[special] = E8M0_NAN
    return codes, scales


def pack_e2m1(codes: np.ndarray) -> np.ndarray:
    """Two E2M1 codes per byte ([Q] §9/§10): element 2k low nibble, 2k+1 high nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_e2m1(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def pack_fp6(codes: np.ndarray) -> np.ndarray:
    """Four 6-bit codes per three bytes: the codes, least significant bit first,
    form one bit stream that is cut into bytes, least significant bit first."""
    c = np.asarray(codes, dtype=np.uint8)
    assert c.shape[-1] % 4 == 0
    bits = np.unpackbits(c[..., None], axis=-1, bitorder="little")[..., :6]   # [..., N, 6]
    stream = bits.reshape(c.shape[:-1] + (c.shape[-1] * 6,))
    return np.packbits(stream, axis=-1, bitorder="little")


def unpack_fp6(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    assert p.shape[-1] % 3 == 0
    stream = np.unpackbits(p, axis=-1, bitorder="little")
    bits = stream.reshape(p.shape[:-1] + (p.shape[-1] * 8 // 6, 6))
    return np.packbits(bits, axis=-1, bitorder="little")[..., 0]


def pack_codes(codes: np.ndarray, fmt: Fmt) -> np.ndarray:
    if fmt.bits == 4:
        return pack_e2m1(codes)
    if fmt.bits == 6:
        return pack_fp6(codes)
    return np.asarray(codes, dtype=np.uint8)


def unpack_codes(packed: np.ndarray, fmt: Fmt) -> np.ndarray:
    if fmt.bits == 4:
        return unpack_e2m1(packed)
    if fmt.bits == 6:
        return unpack_fp6(packed)
    return np.asarray(packed, dtype=np.uint8)


def _quantize_rows(x64: np.ndarray, fmt: Fmt, mode: int):
    b, r, c = x64.shape
    codes, scales = quantize_blocks(x64.reshape(-1, BLOCK), fmt, mode)
    codes = pack_codes(codes.reshape(b, r, c), fmt)
    return codes, scales.reshape(b, r, c // BLOCK)


def quantize(x: np.ndarray, in_dtype: str, fmt: Fmt, mode: int, axis: int) -> dict:
    """Quantize a [B][R][C] (or [R][C]) tensor.

    Row blocks are 32 consecutive elements along C; column blocks are 32
    consecutive rows of one column. The column copy is stored transposed,
    codes [B][C][R] (E2M1: [B][C][R/2], 6-bit: [B][C][3R/4]) and scales [B][C][R/32], so that it
    equals the row-wise quantization of X^T.
    Returns a dict with the keys row_codes/row_scales and/or col_codes/col_scales.
    """
    x64 = widen(x, in_dtype)
    if x64.ndim == 2:
        x64 = x64[None]
    out = {}
    if axis & ROW:
        out["row_codes"], out["row_scales"] = _quantize_rows(x64, fmt, mode)
    if axis & COL:
        xt = np.ascontiguousarray(x64.transpose(0, 2, 1))
        out["col_codes"], out["col_scales"] = _quantize_rows(xt, fmt, mode)
    return out


def round_to_binary(v: np.ndarray, mbits: int, emin: int, emax: int) -> np.ndarray:
    """Round float64 values to a binary format (RNE), returning float64.

    The format has mbits stored mantissa bits, smallest normal exponent emin and
    largest exponent emax; below 2^emin the quantum stays 2^(emin - mbits)
    (gradual underflow). A rounded magnitude above the largest finite value
    overflows to Inf, as IEEE 754 round-to-nearest does.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    finite_nz = np.isfinite(a) & (a > 0)
    safe = np.where(finite_nz, a, 1.0)
    big_e = np.maximum(np.frexp(safe)[1].astype(np.int64) - 1, emin)
    q = np.ldexp(1.0, big_e - mbits)
    r = np.rint(safe / q) * q                      # np.rint rounds halves to even
    maxf = np.ldexp(2.0 - 2.0 ** -mbits, emax)
    r = np.where(r > maxf, np.inf, r)
    r = np.where(finite_nz, r, a)
    return np.copysign(r, v)


def f32_bits(v: np.ndarray) -> np.ndarray:
    r = round_to_binary(v, 23, -126, 127)
    bits = r.astype(np.float32).view(np.uint32).copy()   # exact: r is an FP32 value
    bits[np.isnan(r)] = 0x7FC00000
    return bits


def bf16_bits(v: np.ndarray) -> np.ndarray:
    r = round_to_binary(v, 7, -126, 127)
    bits = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits[np.isnan(r)] = 0x7FC0
    return bits


def dequantize(codes: np.ndarray, scales: np.ndarray, fmt: Fmt, out_dtype: str) -> np.ndarray:
    """Codes + E8M0 scales -> FP32 (uint32 bits) or BF16 (uint16 bits).

    codes: [..., N] (packed: E2M1 [..., N/2], 6-bit [..., 3N/4]); scales: [..., N/32]. Blocks run
    along the last axis, so a transposed column plane dequantizes to X^T.
    [Q] §7: applying an E8M0 scale adds to the exponent, with no rounding
    error, so y = value(code) * 2^(k - 127) is formed exactly in float64 and
    rounded once to the output type. [Q] §2: k = 0xFF makes the whole block NaN.
    """
    c = unpack_codes(codes, fmt)
    k = np.asarray(scales, dtype=np.int64)
    assert c.shape[-1] == k.shape[-1] * BLOCK
    vals = value_table(fmt)[c]
    kk = np.repeat(k, BLOCK, axis=-1)
    y = np.ldexp(vals, np.where(kk == E8M0_NAN, 0, kk - E8M0_BIAS))
    y = np.where(kk == E8M0_NAN, np.nan, y)
    if out_dtype == "f32":
        return f32_bits(y)
    if out_dtype == "bf16":
        return bf16_bits(y)
    raise ValueError(f"unknown output dtype {out_dtype!r}")


def plane_bytes(fmt: Fmt, shape, axis: int):
    """(code bytes, scale bytes) of the requested planes for a [B][R][C] tensor."""
    if len(shape) == 2:
        shape = (1,) + tuple(shape)
    b, r, c = shape
    n = b * r * c
    per = n * fmt.bits // 8
    planes = (1 if axis & ROW else 0) + (1 if axis & COL else 0)
    return per * planes, (n // BLOCK) * planes
