"""MX cast variants: stochastic rounding and 32x32 (2-D) block scaling.

TEST INFRASTRUCTURE, like the rest of ``oracle/``: only the test suite,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` may import it.

What the pages say ([Q] "MXFP4 と NVFP4 は何が違うのか調べてみた", §4, the 4-bit
pretraining recipe): weights use two-dimensional block scaling, and only
gradients use stochastic rounding ([Q] §8 adds that the P3109 draft defines
stochastic rounding among its rounding modes). The pages give neither the
rounding rule in detail nor a random-number source, so the readings below
(listed in the design doc) fix them:

  * Stochastic rounding (SR) of a finite scaled value s with |s| < max: q is
    the element format's spacing at |s| (2^(max(floor(log2|s|), emin) - m) for
    the float formats, 2^-6 for INT8), f = frac(|s| / q), and U is a 16-bit
    random integer; |s| goes up to the next grid value when f > U / 2^16 and
    down otherwise. So P(up) = ceil(f * 2^16) / 2^16 and exact grid values never
    move. |s| >= max saturates, the sign is kept (INT8: two's complement), and
    the shared scale is chosen exactly as for round-to-nearest-even.
  * Random bits: Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random
    numbers: as easy as 1, 2, 3", SC'11), keyed by the 64-bit seed (key word 0
    = low half). Element i of the flat [B][R][C] order of X uses counter
    (g mod 2^32, g >> 32, 0, 0) with g = i >> 3, output word (i >> 1) & 3, and
    its low (i even) or high (i odd) 16 bits. The row and the column copy of
    one element use the same bits.
  * 2-D blocks: X is cut into 32x32 tiles per batch slice; each tile gets one
    E8M0 scale from its largest magnitude, with the same rules as 1x32 blocks
    (NaN/Inf anywhere in the tile -> 0xFF). Row copy: codes [B][R][C'], scales
    [B][R/32][C/32]. Column copy: the same quantization of X^T, codes
    [B][C][R'], scales [B][C/32][R/32] (the transposed scale grid).
"""
from __future__ import annotations

import numpy as np

from .mx_oracle import (BLOCK, COL, E8M0_BIAS, E8M0_NAN, ROW, Fmt, encode_elements, max_finite,
                        pack_codes, shared_exponent, unpack_codes, value_table, widen, bf16_bits,
                        f32_bits)

__all__ = ["philox4x32_10", "sr_bits", "encode_elements_sr", "quantize_ex", "dequantize_2d",
           "RNE", "SR", "BLOCK_1X32", "BLOCK_32X32"]

RNE, SR = "rne", "sr"
BLOCK_1X32, BLOCK_32X32 = "1x32", "32x32"

_M0, _M1 = 0xD2511F53, 0xCD9E8D57      # Philox4x32 multipliers
_W0, _W1 = 0x9E3779B9, 0xBB67AE85      # Weyl key increments
_MASK = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr: np.ndarray, key) -> np.ndarray:
    """Philox4x32 with 10 rounds. ctr: [..., 4] uint32, key: (k0, k1).

    Each round multiplies words 0 and 2 by the two constants (64-bit products),
    and the new state is (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1,
    lo(M0*c0)); the key is bumped by the Weyl constants before every round but
    the first."""
    c = [np.asarray(ctr[..., j], dtype=np.uint64) for j in range(4)]
    k0, k1 = np.uint64(key[0] & 0xFFFFFFFF), np.uint64(key[1] & 0xFFFFFFFF)
    for r in range(10):
        if r:
            k0 = (k0 + np.uint64(_W0)) & _MASK
            k1 = (k1 + np.uint64(_W1)) & _MASK
        p0 = np.uint64(_M0) * c[0]
        p1 = np.uint64(_M1) * c[2]
        c = [(p1 >> np.uint64(32)) ^ c[1] ^ k0, p1 & _MASK, (p0 >> np.uint64(32)) ^ c[3] ^ k1, p0 & _MASK]
    return np.stack([v.astype(np.uint32) for v in c], axis=-1)


def sr_bits(seed: int, n: int, start: int = 0) -> np.ndarray:
    """16 random bits for each of the flat elements start .. start+n-1 (uint16 [n])."""
    g0 = start >> 3
    ng = ((start + n + 7) >> 3) - g0
    g = np.arange(g0, g0 + ng, dtype=np.uint64)
    ctr = np.stack([g & _MASK, g >> np.uint64(32), np.zeros_like(g), np.zeros_like(g)], axis=-1)
    words = philox4x32_10(ctr, (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))   # [ng, 4]
    halves = np.stack([words & 0xFFFF, words >> 16], axis=-1).astype(np.uint16)   # [ng, 4, 2]
    off = start - 8 * g0
    return halves.reshape(-1)[off:off + n]


def _spacing(a: np.ndarray, fmt: Fmt) -> np.ndarray:
    """Grid spacing of the element format at magnitudes a (> 0)."""
    if fmt.integer:
        return np.full_like(a, 2.0 ** -fmt.bias)
    emin = 1 - fmt.bias
    big_e = np.frexp(a)[1].astype(np.int64) - 1                 # floor(log2 a)
    return np.ldexp(1.0, np.maximum(big_e, emin) - fmt.mbits)


def encode_elements_sr(s: np.ndarray, fmt: Fmt, u16: np.ndarray) -> np.ndarray:
    """Element codes of finite scaled values s under stochastic rounding."""
    s = np.asarray(s, dtype=np.float64)
    a = np.abs(s)
    vmax = max_finite(fmt)
    nz = a > 0
    q = _spacing(np.where(nz, a, 1.0), fmt)
    x = a / q                                                   # exact: q is a power of two
    n = np.floor(x)
    f = x - n
    up = f > np.asarray(u16, dtype=np.float64) / 65536.0
    mag = (n + up) * q
    mag = np.where(a >= vmax, vmax, mag)
    mag = np.where(nz, mag, 0.0)
    return encode_elements(np.copysign(mag, s), fmt)            # mag is a grid value: its own code


def _quant_plane(x64: np.ndarray, u: np.ndarray | None, fmt: Fmt, mode: int, block: str):
    b, r, c = x64.shape
    if block == BLOCK_1X32:
        blocks = x64.reshape(b, r, c // BLOCK, BLOCK)
        axes = (3,)
    elif block == BLOCK_32X32:
        assert r % BLOCK == 0
        blocks = x64.reshape(b, r // BLOCK, BLOCK, c // BLOCK, BLOCK).transpose(0, 1, 3, 2, 4)
        axes = (3, 4)
    else:
        raise ValueError(f"unknown block shape {block!r}")
    special = ~np.isfinite(blocks).all(axis=axes)
    clean = np.where(np.isfinite(blocks), blocks, 0.0)
    amax = np.max(np.abs(clean), axis=axes)
    e = shared_exponent(amax.reshape(-1), fmt, mode).reshape(amax.shape)
    e_el = e.reshape(e.shape + (1,) * len(axes))
    s = np.ldexp(clean, -e_el)                                  # exact: division by 2^e
    if u is None:
        codes = encode_elements(s, fmt)
    else:
        ub = u.reshape(b, r, c // BLOCK, BLOCK) if block == BLOCK_1X32 else \
            u.reshape(b, r // BLOCK, BLOCK, c // BLOCK, BLOCK).transpose(0, 1, 3, 2, 4)
        codes = encode_elements_sr(s, fmt, ub)
    sp = special.reshape(special.shape + (1,) * len(axes))
    codes = np.where(sp, 0x7F if fmt.has_nan else 0x0, codes).astype(np.uint8)
    scales = np.where(special, E8M0_NAN, e + E8M0_BIAS).astype(np.uint8)
    if block == BLOCK_32X32:
        codes = codes.transpose(0, 1, 3, 2, 4)
    codes = pack_codes(codes.reshape(b, r, c), fmt)
    return codes, scales                                        # scales [b, r, c/32] or [b, r/32, c/32]


def quantize_ex(x: np.ndarray, in_dtype: str, fmt: Fmt, mode: int, axis: int, rounding: str = RNE,
                seed: int = 0, block: str = BLOCK_1X32, first: int = 0) -> dict:
    """quantize() with a rounding rule (RNE or SR) and a block shape (1x32 or 32x32).

    With RNE and 1x32 blocks it computes exactly what mx_oracle.quantize does.
    Returns row_codes/row_scales and/or col_codes/col_scales; the column copy is
    the same quantization of X^T, with each element keeping its random bits.
    ``first`` is the flat index of x's first element in a larger tensor of which
    x is a run of whole rows (its SR draws follow that tensor's order).
    """
    x64 = widen(x, in_dtype)
    if x64.ndim == 2:
        x64 = x64[None]
    u = None
    if rounding == SR:
        u = sr_bits(seed, x64.size, first).reshape(x64.shape)
    elif rounding != RNE:
        raise ValueError(f"unknown rounding {rounding!r}")
    out = {}
    if axis & ROW:
        out["row_codes"], out["row_scales"] = _quant_plane(x64, u, fmt, mode, block)
    if axis & COL:
        xt = np.ascontiguousarray(x64.transpose(0, 2, 1))
        ut = None if u is None else np.ascontiguousarray(u.transpose(0, 2, 1))
        out["col_codes"], out["col_scales"] = _quant_plane(xt, ut, fmt, mode, block)
    return out


def dequantize_2d(codes: np.ndarray, scales: np.ndarray, fmt: Fmt, out_dtype: str) -> np.ndarray:
    """Codes [..., R, C'] with 32x32-block scales [..., R/32, C/32] -> FP32 / BF16 bits.
    Same arithmetic as dequantize(): value(code) * 2^(k-127) exactly, one rounding."""
    c = unpack_codes(codes, fmt)
    k = np.asarray(scales, dtype=np.int64)
    kk = np.repeat(np.repeat(k, BLOCK, axis=-1), BLOCK, axis=-2)
    assert kk.shape == c.shape
    vals = value_table(fmt)[c]
    y = np.ldexp(vals, np.where(kk == E8M0_NAN, 0, kk - E8M0_BIAS))
    y = np.where(kk == E8M0_NAN, np.nan, y)
    if out_dtype == "f32":
        return f32_bits(y)
    if out_dtype == "bf16":
        return bf16_bits(y)
    raise ValueError(f"unknown output dtype {out_dtype!r}")
