"""Pins of the oracle's element and scale formats against what the pages print
and against independent library decoders (torch's float8 types)."""
import math

import numpy as np
import pytest
import torch

import oracle as O


def test_e2m1_value_table_matches_page():
    # "MXFP4 と NVFP4 は何が違うのか調べてみた" §1: 16 patterns, non-negative values
    # 0, 0.5, 1, 1.5, 2, 3, 4, 6, the negative side mirrors them, 15 distinct
    # values (+-0), no Inf and no NaN, largest value 6.
    t = O.value_table(O.E2M1)
    assert t.shape == (16,)
    assert t[:8].tolist() == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert t[8:].tolist() == [-v for v in t[:8].tolist()]
    assert np.signbit(t[8])
    assert len(set(t.tolist())) == 15
    assert np.isfinite(t).all()
    assert O.max_finite(O.E2M1) == 6.0
    # the gpt-oss news article: 8 positive and 8 negative encodings
    assert int((~np.signbit(t)).sum()) == 8 and int(np.signbit(t).sum()) == 8


def test_e4m3_max_is_448():
    # Same article §3: the E4M3 maximum is 448 (also the NVFP4 global-scale divisor 6 * 448).
    assert O.max_finite(O.E4M3) == 448.0
    t = O.value_table(O.E4M3)
    assert int(np.nanargmax(np.where(np.isnan(t), -1, t))) == 0x7E


@pytest.mark.parametrize("fmt,tdt", [(O.E4M3, torch.float8_e4m3fn), (O.E5M2, torch.float8_e5m2)])
def test_fp8_tables_match_torch(fmt, tdt):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(tdt).to(torch.float64).numpy()
    ours = O.value_table(fmt)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_e5m2_specials():
    t = O.value_table(O.E5M2)
    assert t[0x7C] == math.inf and t[0xFC] == -math.inf
    assert all(np.isnan(t[c]) for c in (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF))
    assert O.max_finite(O.E5M2) == 57344.0


def test_emax_values():
    # §4 of the same article: the OCP example rule subtracts 2 (E2M1's largest binade).
    assert O.emax_of(O.E2M1) == 2
    assert O.emax_of(O.E4M3) == 8
    assert O.emax_of(O.E5M2) == 15


def test_bits_per_element():
    # §2 tables: MXFP4 = 32 x 4 + 8 = 136 bits per block = 4.25 bits/element;
    # MXFP8 = 8.25 bits/element.
    for fmt, bpe in ((O.E2M1, 4.25), (O.E4M3, 8.25), (O.E5M2, 8.25)):
        cb, sb = O.plane_bytes(fmt, (1, 64, 4096), O.ROW)
        assert (cb + sb) * 8 / (64 * 4096) == bpe
        cb2, sb2 = O.plane_bytes(fmt, (1, 64, 4096), O.BOTH)
        assert (cb2, sb2) == (2 * cb, 2 * sb)


def test_tile_footprint_matches_page():
    # §10 table: a 64x64 weight tile kept 4-bit packed takes 2 KB plus 128 bytes of scales.
    cb, sb = O.plane_bytes(O.E2M1, (64, 64), O.ROW)
    assert (cb, sb) == (2048, 128)


def test_e8m0_range_and_nan_scale():
    # §2: codes 0..254 <-> 2^-127 .. 2^127, 0xFF = NaN (no Inf); a NaN scale makes
    # all 32 elements of the block NaN. Element 1.0 in E4M3 is code 0x38.
    codes = np.full((256, 32), 0x38, dtype=np.uint8)
    scales = np.arange(256, dtype=np.uint8).reshape(256, 1)
    y = O.dequantize(codes, scales, O.E4M3, "f32").view(np.float32)
    for k in range(255):
        assert (y[k] == np.float32(math.ldexp(1.0, k - 127))).all(), k
    assert np.isnan(y[255]).all()
    assert (O.dequantize(codes, scales, O.E4M3, "f32")[255] == 0x7FC00000).all()
