"""FP4-in-FP8 nested requantization: MXFP4 weights re-expressed as FP8 E4M3 with
one scale per 128x128 block, and the scale-ratio check for losslessness.

TEST INFRASTRUCTURE, like the rest of ``oracle/``: only the test suite,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` may import it.

What the pages say ([Q] "MXFP4 と NVFP4 は何が違うのか調べてみた", §6, DeepSeek-V4's
nested structure, and the closing notes on figures): FP32 master weights are
quantized to MXFP4 (1x32 tiles with E8M0 scales) and then dequantized into FP8
E4M3 for the existing FP8 training path, whose scales are per 128x128 tile; a
128x128 tile holds 4 x 128 = 512 of the 1x32 tiles. E4M3 has two more exponent
bits than E2M1, so the conversion is lossless as long as, inside each 128x128
tile, the ratio of the largest to the smallest 1x32 scale stays under a
threshold; this is a property of the weights, observed, not guaranteed, and the
pages ask for it to be checked.

The pages give neither the FP8 block scale nor the threshold. The readings
(listed in the design doc) fix them:

  * A 1x32 sub-block is *active* when one of its codes has a nonzero magnitude
    and its scale is not the NaN code 0xFF. Only active sub-blocks enter the
    block's largest and smallest scale codes kmax and kmin (an all-zero tile's
    scale carries no information; a NaN tile has no magnitude).
  * The FP8 block scale is the power of two S = 2^(kmax - 133): the largest
    E2M1 magnitude 6 of the largest sub-block lands on 6 * 2^6 = 384 <= 448.
    With no active sub-block, S = 1.
  * Each element v = e2m1 * 2^(k - 127) is stored as the E4M3 code of v / S,
    rounded to nearest-even (exact whenever v / S is an E4M3 value); a NaN
    sub-block stores 0x7F; zeros keep their sign.
  * The check reports spread = kmax - kmin per 128x128 block (0 with fewer
    than two active sub-blocks). v / S = e2m1 * 2^E with E = k - kmax + 6; every
    E2M1 value times 2^E is an E4M3 value for -8 <= E <= 6, so spread <= 14
    guarantees a lossless block (the threshold: a scale ratio of 2^14). At
    spread 15 the E2M1 values 0.5 and 1.5 of the smallest sub-blocks no longer
    fit (0.5 * 2^-9 and 1.5 * 2^-9 fall between E4M3's subnormal steps).
  * Blocks at a ragged edge (rows or columns not a multiple of 128) cover what
    is there. Layout: E4M3 codes [B][R][C]; block scales and spreads
    [B][ceil(R/128)][ceil(C/128)]; the transposed copy is the same codes as
    [B][C][R] with the transposed scale grid (the blocks are square, so the
    transposed weight needs no new quantization).
"""
from __future__ import annotations

import numpy as np

from .mx_oracle import BLOCK, E2M1, E4M3, E8M0_BIAS, E8M0_NAN, encode_elements, unpack_e2m1, value_table

__all__ = ["FP8_BLOCK", "SUBS_PER_FP8_BLOCK", "LOSSLESS_SPREAD", "requant_fp4_to_fp8", "dequantize_fp8_blocks"]

FP8_BLOCK = 128                                  # [Q] §6: 128 x 128 FP8 tiles
SUBS_PER_FP8_BLOCK = FP8_BLOCK * FP8_BLOCK // BLOCK   # 512 1x32 tiles ([Q] §6: 4 x 128)
SHIFT = 6                                        # E2M1 max 6 lands on 6 * 2^6 = 384
LOSSLESS_SPREAD = 14                             # E in [-8, 6]: 6 - (-8)


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def _active(qs: np.ndarray, k: np.ndarray) -> np.ndarray:
    """Sub-blocks with a nonzero magnitude code and a finite (non-NaN) scale."""
    return ((qs & 0x7) != 0).any(axis=-1) & (k != E8M0_NAN)


def requant_fp4_to_fp8(codes: np.ndarray, scales: np.ndarray) -> dict:
    """MXFP4 plane -> FP8 E4M3 codes with 128x128 block scales.

    codes: packed E2M1 [B][R][C/2] (or [R][C/2]); scales: E8M0 [B][R][C/32].
    Returns e4m3 [B][R][C] uint8, block_scale [B][R'][C'] float32 (R' =
    ceil(R/128), C' = ceil(C/128)), spread [B][R'][C'] uint8, and the
    transposed copy e4m3_t [B][C][R] with block_scale_t / spread_t [B][C'][R'].
    """
    squeeze = np.asarray(codes).ndim == 2
    q = unpack_e2m1(np.asarray(codes, dtype=np.uint8))
    k = np.asarray(scales, dtype=np.int64)
    if squeeze:
        q, k = q[None], k[None]
    b, r, c = q.shape
    ns = c // BLOCK
    assert k.shape == (b, r, ns)
    qs = q.reshape(b, r, ns, BLOCK)
    active = _active(qs, k)                                              # [b, r, ns]

    # kmax / kmin over the active sub-blocks of each 128x128 block
    nbr, nbc = _ceil_div(r, FP8_BLOCK), _ceil_div(c, FP8_BLOCK)
    spb = FP8_BLOCK // BLOCK                                             # 4 sub-blocks per block row
    pad_r, pad_s = nbr * FP8_BLOCK - r, nbc * spb - ns
    act = np.pad(active, ((0, 0), (0, pad_r), (0, pad_s)))
    kk = np.pad(k, ((0, 0), (0, pad_r), (0, pad_s)))
    act = act.reshape(b, nbr, FP8_BLOCK, nbc, spb)
    kk = kk.reshape(b, nbr, FP8_BLOCK, nbc, spb)
    any_act = act.any(axis=(2, 4))
    kmax = np.where(act, kk, -1).max(axis=(2, 4))
    kmin = np.where(act, kk, 1 << 20).min(axis=(2, 4))
    kmax = np.where(any_act, kmax, E8M0_BIAS + SHIFT)                    # S = 1 for an empty block
    spread = np.where(any_act, kmax - kmin, 0).astype(np.uint8)
    s_exp = kmax - E8M0_BIAS - SHIFT                                     # S = 2^s_exp
    block_scale = np.ldexp(np.float32(1), s_exp).astype(np.float32)

    # every element: v / S = e2m1 * 2^(k - 127 - s_exp), rounded to E4M3
    kmax_el = np.repeat(np.repeat(kmax, FP8_BLOCK, axis=1), spb, axis=2)[:, :r, :ns]
    shift = k - kmax_el + SHIFT                                          # E per sub-block
    vals = value_table(E2M1)[qs]                                         # exact, signed zeros kept
    scaled = vals * np.ldexp(1.0, np.clip(shift, -300, 300))[..., None]  # exact in float64
    e4 = encode_elements(scaled, E4M3)
    e4 = np.where((k == E8M0_NAN)[..., None], 0x7F, e4).astype(np.uint8).reshape(b, r, c)

    out = {"e4m3": e4, "block_scale": block_scale, "spread": spread,
           "e4m3_t": np.ascontiguousarray(e4.transpose(0, 2, 1)),
           "block_scale_t": np.ascontiguousarray(block_scale.transpose(0, 2, 1)),
           "spread_t": np.ascontiguousarray(spread.transpose(0, 2, 1))}
    if squeeze:
        out = {key: v[0] for key, v in out.items()}
    return out


def dequantize_fp8_blocks(e4m3: np.ndarray, block_scale: np.ndarray) -> np.ndarray:
    """E4M3 codes [..., R, C] with 128x128 block scales [..., R', C'] -> float64 values."""
    e4m3 = np.asarray(e4m3)
    r, c = e4m3.shape[-2:]
    s = np.asarray(block_scale, dtype=np.float64)
    s = np.repeat(np.repeat(s, FP8_BLOCK, axis=-2), FP8_BLOCK, axis=-1)[..., :r, :c]
    return value_table(E4M3)[e4m3] * s
