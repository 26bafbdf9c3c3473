"""Pins of the oracle's MXFP6 (E2M3, E3M2) and MXINT8 elements.

The pages list these formats in the MX family table ("MXFP4 と NVFP4 は何が違う
のか調べてみた" §2: MXFP6 = E2M3 or E3M2 at 6.25 bits per element, MXINT8 = INT8
at 8.25) without printing their bit layouts. Independent references here:
  * E2M3 is E4M3's four lowest binades moved up by 2^6, and E3M2 is E5M2's
    eight lowest binades moved up by 2^12 (same mantissa width, subnormal
    quantum and bias offset), so torch's float8 decoders and its RNE float8
    casts give every value and every rounding decision;
  * INT8 codes are two's-complement bytes (numpy's int8 view) read as k / 64,
    and its rounding is numpy's rint followed by a clip;
  * the 6-bit packing is checked against a closed form over Python integers.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O

CARRIER = {"e2m3": (torch.float8_e4m3fn, 6), "e3m2": (torch.float8_e5m2, 12)}


def fp6_from_fp8(c8: np.ndarray) -> np.ndarray:
    """An FP8 code of magnitude <= 0x1F -> the 6-bit code with the same low 5 bits."""
    c8 = np.asarray(c8, dtype=np.int64)
    mag = c8 & 0x7F
    assert (mag <= 0x1F).all()
    return (((c8 >> 7) & 1) << 5 | mag).astype(np.uint8)


def fp8_from_fp6(c6: np.ndarray) -> np.ndarray:
    c6 = np.asarray(c6, dtype=np.int64)
    return (((c6 >> 5) & 1) << 7 | (c6 & 0x1F)).astype(np.uint8)


def test_family_bits_per_element():
    # §2 family table: MXFP6 6.25 and MXINT8 8.25 bits per element.
    for fmt, bpe in ((O.E2M3, 6.25), (O.E3M2, 6.25), (O.INT8, 8.25)):
        cb, sb = O.plane_bytes(fmt, (1, 64, 4096), O.ROW)
        assert (cb + sb) * 8 / (64 * 4096) == bpe


@pytest.mark.parametrize("name", ["e2m3", "e3m2"])
def test_fp6_tables_are_fp8_low_binades(name):
    fmt = O.FORMATS[name]
    tdt, shift = CARRIER[name]
    codes = np.arange(64)
    c8 = torch.from_numpy(fp8_from_fp6(codes)).view(tdt).to(torch.float64).numpy()
    ref = np.ldexp(c8, shift)
    ours = O.value_table(fmt)
    assert np.isfinite(ours).all()                            # no Inf, no NaN
    assert np.array_equal(ours, ref)
    assert np.array_equal(np.signbit(ours), np.signbit(ref))
    assert len(set(ours.tolist())) == 63                      # +-0 coincide
    assert O.max_finite(fmt) == {"e2m3": 7.5, "e3m2": 28.0}[name]
    assert O.emax_of(fmt) == {"e2m3": 2, "e3m2": 4}[name]


def test_int8_table_is_twos_complement_over_64():
    t = O.value_table(O.INT8)
    ref = np.arange(256, dtype=np.int64).astype(np.uint8).view(np.int8).astype(np.float64) / 64.0
    assert np.array_equal(t, ref)
    assert O.max_finite(O.INT8) == 127 / 64
    assert O.emax_of(O.INT8) == 0


def _all_bf16_finite():
    bits = np.arange(1 << 16, dtype=np.uint32)
    bits = bits[(bits & 0x7FFF) < 0x7F80]
    return (bits << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("name", ["e2m3", "e3m2"])
def test_fp6_encoder_exhaustive_vs_torch(name):
    """Every finite BF16 pattern divided by every E8M0 scale 2^e: the oracle's
    code equals torch's RNE float8 cast of the value clamped to +-max and moved
    down by the carrier shift."""
    fmt = O.FORMATS[name]
    tdt, shift = CARRIER[name]
    x = _all_bf16_finite()
    vmax = O.max_finite(fmt)
    for e in range(-127, 128):
        s = np.ldexp(x, -e)
        ours = O.encode_elements(s, fmt)
        moved = np.ldexp(np.clip(s, -vmax, vmax), -shift).astype(np.float32)
        ref = fp6_from_fp8(torch.from_numpy(moved).to(tdt).view(torch.uint8).numpy())
        bad = np.nonzero(ours != ref)[0]
        assert bad.size == 0, (e, s[bad[:5]], ours[bad[:5]], ref[bad[:5]])


def test_int8_encoder_exhaustive_vs_numpy_rint():
    x = _all_bf16_finite()
    for e in range(-127, 128):
        s = np.ldexp(x, -e)
        ours = O.encode_elements(s, O.INT8)
        ref = np.clip(np.rint(s * 64.0), -127, 127).astype(np.int8).view(np.uint8)
        assert np.array_equal(ours, ref), e


def brute_int8(s: float) -> int:
    """Nearest of the 255 codes -127..127 (k / 64); ties -> even k."""
    s = min(max(s, -2.5), 2.5)            # keeps distances exact; beyond +-2 nothing changes
    best, best_d = None, None
    for k in range(-127, 128):
        d = abs(k / 64.0 - s)
        if best is None or d < best_d or (d == best_d and k % 2 == 0):
            best, best_d = k, d
    return best & 0xFF


def test_int8_encoder_matches_brute_force_scan():
    pts = [k / 64.0 for k in range(128)] + [(k + 0.5) / 64.0 for k in range(128)]
    pts += [2.0, 2.5, 100.0, 1e30]
    probes = []
    for p in pts:
        probes += [p, math.nextafter(p, math.inf), math.nextafter(p, 0.0)]
    probes += [-p for p in probes] + [0.0, -0.0]
    got = O.encode_elements(np.array(probes), O.INT8)
    assert got.tolist() == [brute_int8(p) for p in probes]


def test_int8_saturation_and_zero():
    enc = lambda v: int(O.encode_elements(np.array([v]), O.INT8)[0])
    assert enc(2.0) == 0x7F and enc(-2.0) == 0x81          # symmetric: -128 never produced
    assert enc(127.5 / 64) == 0x7F                          # tie 127.5 -> 128 -> clipped
    assert enc(126.5 / 64) == 126 and enc(-126.5 / 64) == (-126) & 0xFF
    assert enc(-0.0) == 0 and enc(-0.25 / 64) == 0
    assert enc(1 / 128) == 0 and enc(3 / 128) == 2         # ties to even integers


def test_fp6_saturation():
    for name, vmax, top in (("e2m3", 7.5, 0x1F), ("e3m2", 28.0, 0x1F)):
        fmt = O.FORMATS[name]
        enc = lambda v: int(O.encode_elements(np.array([v]), fmt)[0])
        assert enc(vmax) == top and enc(vmax * 1.07) == top and enc(1e9) == top
        assert enc(-1e9) == top | 0x20
        assert enc(-0.0) == 0x20


def test_fp6_packing_closed_form():
    rng = np.random.default_rng(11)
    codes = rng.integers(0, 64, size=(5, 96), dtype=np.uint8)
    packed = O.pack_fp6(codes)
    assert packed.shape == (5, 72)
    for r in range(5):
        for g in range(24):
            c = [int(v) for v in codes[r, 4 * g:4 * g + 4]]
            word = int.from_bytes(bytes(packed[r, 3 * g:3 * g + 3].tolist()), "little")
            assert word == c[0] | c[1] << 6 | c[2] << 12 | c[3] << 18
    assert np.array_equal(O.unpack_fp6(packed), codes)
    one = lambda i: O.pack_fp6(np.array([0x3F if j == i else 0 for j in range(4)], np.uint8)).tolist()
    assert one(0) == [0x3F, 0x00, 0x00]
    assert one(1) == [0xC0, 0x0F, 0x00]
    assert one(2) == [0x00, 0xF0, 0x03]
    assert one(3) == [0x00, 0x00, 0xFC]


def test_plane_shapes_for_new_formats():
    x = np.linspace(-3, 3, 64 * 96, dtype=np.float32).reshape(64, 96)
    out = O.quantize(x, "f32", O.E3M2, O.ROUNDUP, O.BOTH)
    assert out["row_codes"].shape == (1, 64, 72) and out["row_scales"].shape == (1, 64, 3)
    assert out["col_codes"].shape == (1, 96, 48) and out["col_scales"].shape == (1, 96, 2)
    out = O.quantize(x, "f32", O.INT8, O.FLOOR, O.ROW)
    assert out["row_codes"].shape == (1, 64, 96)
    y = O.dequantize(out["row_codes"], out["row_scales"], O.INT8, "f32").view(np.float32)
    assert np.abs(y - x).max() <= 3 / 128 + 1e-7    # scale 2^1, quantum 2 / 64, half of it
