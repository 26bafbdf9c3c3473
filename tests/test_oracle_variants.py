"""Pins of the oracle's stochastic rounding, its random bits and 32x32 blocks.

Independent references:
  * Philox4x32-10 known-answer vectors published with the Random123 library
    (Salmon et al., SC'11), for three (counter, key) pairs;
  * for stochastic rounding, brute-force scans of every code (round toward and
    away from zero are its two extreme random draws), the exact count of
    "up" draws over all 2^16 random values (a closed form in rationals), and
    numpy's floor/ceil for INT8;
  * for 2-D blocks, the 1-D quantization (pinned elsewhere): a 32x32 tile's
    scale is the largest of its 32 row-block scales, equal rows reduce to 1-D,
    and the column copy is the transpose.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

FMTS = [O.E4M3, O.E5M2, O.E2M1, O.E2M3, O.E3M2, O.INT8]


# ---------------- Philox4x32-10 ----------------

KAT = [  # (counter, key, output) from the Random123 known-answer tests
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,out", KAT)
def test_philox_known_answers(ctr, key, out):
    got = O.philox4x32_10(np.array([ctr], dtype=np.uint32), key)[0]
    assert [int(v) for v in got] == list(out)


def test_sr_bits_layout_against_known_answer():
    # seed 0, elements 0..7 use counter 0: the zero-key answer, low half first
    w = KAT[0][2]
    exp = [h for v in w for h in (v & 0xFFFF, v >> 16)]
    assert O.sr_bits(0, 8).tolist() == exp
    # the seed is the key: key (0xFFFFFFFF, 0xFFFFFFFF) with counter 0 differs from seed 0
    assert O.sr_bits((1 << 64) - 1, 8).tolist() != exp
    # element 8 starts counter 1; a window of the stream is the same bits
    assert O.sr_bits(0, 16)[:8].tolist() == exp
    assert np.array_equal(O.sr_bits(7, 40)[5:29], O.sr_bits(7, 24, start=5))


# ---------------- stochastic rounding ----------------

def grid(fmt):
    """Magnitudes the encoder can produce (INT8's -128 is never produced)."""
    vals = sorted(set(abs(O.decode_code(fmt, c)) for c in range(1 << fmt.bits)
                      if math.isfinite(O.decode_code(fmt, c)) and not (fmt.integer and c == 0x80)))
    return vals


def brute_toward_zero(s, fmt):
    a = min(abs(s), O.max_finite(fmt))
    return max(v for v in grid(fmt) if v <= a)


def brute_away_from_zero(s, fmt):
    a = min(abs(s), O.max_finite(fmt))
    return min(v for v in grid(fmt) if v >= a)


def probes(fmt):
    g = grid(fmt)
    pts = [(x + y) / 2 for x, y in zip(g[:-1], g[1:])] + [x * 0.9 + y * 0.1 for x, y in zip(g[:-1], g[1:])]
    pts += g + [g[-1] * 1.01, g[-1] * 3, g[1] * 0.37, g[1] * 1e-6]
    return [p for p in pts] + [-p for p in pts]


def decoded(codes, fmt):
    return O.value_table(fmt)[np.asarray(codes, dtype=np.int64)]


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_sr_extreme_draws_are_directed_roundings(fmt):
    """U = 0 rounds every non-grid magnitude away from zero; U = 65535 rounds it
    toward zero unless frac > 65535/65536."""
    s = np.array(probes(fmt))
    up = decoded(O.encode_elements_sr(s, fmt, np.zeros(len(s), np.uint16)), fmt)
    dn = decoded(O.encode_elements_sr(s, fmt, np.full(len(s), 0xFFFF, np.uint16)), fmt)
    for v, a, b in zip(s, up, dn):
        assert abs(a) == brute_away_from_zero(v, fmt), v
        assert abs(b) == brute_toward_zero(v, fmt), v
        assert math.copysign(1, a) == math.copysign(1, v) or a == 0 and fmt.integer


@pytest.mark.parametrize("fmt", [O.E2M1, O.E4M3, O.INT8], ids=lambda f: f.name)
def test_sr_up_count_over_all_draws(fmt):
    """Over all 2^16 values of U, the number of draws that round up is
    ceil(f * 2^16) for f = (|s| - lo) / (hi - lo), in exact rationals."""
    u = np.arange(1 << 16, dtype=np.uint16)
    g = grid(fmt)
    for lo, hi in zip(g[:-1], g[1:]):
        for w in (Fraction(1, 3), Fraction(1, 2), Fraction(5, 7), Fraction(1, 1 << 20)):
            s = Fraction(lo) + (Fraction(hi) - Fraction(lo)) * w
            sf = float(s)
            f = (Fraction(sf) - Fraction(lo)) / (Fraction(hi) - Fraction(lo))
            codes = O.encode_elements_sr(np.full(len(u), sf), fmt, u)
            n_up = int(np.sum(decoded(codes, fmt) == hi))
            n_dn = int(np.sum(decoded(codes, fmt) == lo))
            assert n_up + n_dn == len(u)
            assert n_up == math.ceil(f * (1 << 16)), (lo, hi, w)


def test_sr_leaves_grid_values_and_saturates():
    u = np.random.default_rng(1).integers(0, 1 << 16, size=64).astype(np.uint16)
    for fmt in FMTS:
        codes = np.array([c for c in range(1 << fmt.bits) if math.isfinite(O.decode_code(fmt, c))
                          and not (fmt.integer and c == 0x80)])
        vals = decoded(codes, fmt)
        for k in range(0, len(codes), 64):
            v = vals[k:k + 64]
            got = O.encode_elements_sr(v, fmt, u[:len(v)])
            assert np.array_equal(decoded(got, fmt), v), fmt.name
        big = np.array([O.max_finite(fmt) * 1.5, -O.max_finite(fmt) * 1.01])
        got = decoded(O.encode_elements_sr(big, fmt, np.zeros(2, np.uint16)), fmt)
        assert got.tolist() == [O.max_finite(fmt), -O.max_finite(fmt)]


def test_sr_int8_matches_numpy_floor():
    rng = np.random.default_rng(2)
    s = rng.uniform(-2.2, 2.2, 20000)
    u = rng.integers(0, 1 << 16, 20000).astype(np.uint16)
    a = np.abs(s) * 64
    f = a - np.floor(a)
    k = np.floor(a) + (f > u / 65536.0)
    k = np.minimum(k, 127) * np.sign(s)
    ref = k.astype(np.int64).astype(np.int8).view(np.uint8)
    assert np.array_equal(O.encode_elements_sr(s, O.INT8, u), ref)


def test_sr_quantize_is_unbiased_over_seeds():
    """The mean of the dequantized SR results over many seeds approaches x (with
    the round-up scale rule, so nothing is clipped)."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((32, 64)) * 0.3).astype(np.float32)
    acc = np.zeros(x.shape)
    n = 400
    for seed in range(n):
        q = O.quantize_ex(x, "f32", O.E2M1, O.ROUNDUP, O.ROW, rounding=O.SR, seed=seed)
        acc += O.dequantize(q["row_codes"][0], q["row_scales"][0], O.E2M1, "f32").view(np.float32)
    mean = acc / n
    rne = O.quantize(x, "f32", O.E2M1, O.ROUNDUP, O.ROW)
    # one SR step size per element: the block scale times the local E2M1 spacing (<= 2)
    step = np.ldexp(2.0, rne["row_scales"][0].astype(int) - 127).repeat(32, axis=1)
    assert np.all(np.abs(mean - x) <= 4 * step / math.sqrt(n) + 1e-12)
    assert np.abs(mean - x).mean() < np.abs(O.dequantize(rne["row_codes"][0], rne["row_scales"][0], O.E2M1,
                                                          "f32").view(np.float32) - x).mean()


def test_sr_column_copy_uses_the_elements_bits():
    """The column copy of X with SR equals the SR row copy of X^T built from the
    same per-element bits (X's flat order), not from X^T's own order."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((64, 96)).astype(np.float32)
    q = O.quantize_ex(x, "f32", O.E4M3, O.FLOOR, O.COL, rounding=O.SR, seed=9)
    u = O.sr_bits(9, x.size).reshape(x.shape).T
    xt = x.T.astype(np.float64)
    codes = []
    scales = O.quantize(np.ascontiguousarray(x.T), "f32", O.E4M3, O.FLOOR, O.ROW)["row_scales"][0]
    e = scales.astype(int).repeat(32, axis=1) - 127
    codes = O.encode_elements_sr(np.ldexp(xt, -e), O.E4M3, u)
    assert np.array_equal(q["col_codes"][0], codes)
    assert np.array_equal(q["col_scales"][0], scales)


def test_sr_rne_and_sr_share_scales():
    x = np.random.default_rng(5).standard_normal((64, 128)).astype(np.float32)
    for fmt in FMTS:
        a = O.quantize_ex(x, "f32", fmt, O.ROUNDUP, O.BOTH, rounding=O.SR, seed=1)
        b = O.quantize(x, "f32", fmt, O.ROUNDUP, O.BOTH)
        assert np.array_equal(a["row_scales"], b["row_scales"])
        assert np.array_equal(a["col_scales"], b["col_scales"])


# ---------------- 32x32 blocks ----------------

def tiles_input(seed=6, b=2, r=96, c=128):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((b, r, c)) * np.exp2(rng.integers(-6, 6, size=(b, r, 1)))
    return x.astype(np.float32)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
@pytest.mark.parametrize("mode", [O.FLOOR, O.ROUNDUP], ids=["floor", "roundup"])
def test_2d_scale_is_max_of_row_block_scales(fmt, mode):
    x = tiles_input()
    q2 = O.quantize_ex(x, "f32", fmt, mode, O.BOTH, block=O.BLOCK_32X32)
    q1 = O.quantize(x, "f32", fmt, mode, O.ROW)["row_scales"]            # [b, r, c/32]
    b, r, c = x.shape
    exp = q1.reshape(b, r // 32, 32, c // 32).max(axis=2)
    assert np.array_equal(q2["row_scales"], exp)
    assert np.array_equal(q2["col_scales"], exp.transpose(0, 2, 1))


@pytest.mark.parametrize("fmt", [O.E4M3, O.INT8, O.E5M2], ids=lambda f: f.name)
def test_2d_column_copy_is_the_transpose(fmt):
    x = tiles_input(7)
    q = O.quantize_ex(x, "f32", fmt, O.FLOOR, O.BOTH, block=O.BLOCK_32X32)
    assert np.array_equal(q["col_codes"], q["row_codes"].transpose(0, 2, 1))


def test_2d_equal_rows_reduce_to_1d():
    row = np.random.default_rng(8).standard_normal((1, 1, 128)).astype(np.float32)
    x = np.repeat(row, 64, axis=1)
    for fmt in FMTS:
        q2 = O.quantize_ex(x, "f32", fmt, O.FLOOR, O.ROW, block=O.BLOCK_32X32)
        q1 = O.quantize(x, "f32", fmt, O.FLOOR, O.ROW)
        assert np.array_equal(q2["row_codes"], q1["row_codes"])
        assert np.array_equal(q2["row_scales"], q1["row_scales"][:, ::32])


def test_2d_specials_poison_one_tile():
    x = tiles_input(9, b=1)
    x[0, 40, 70] = np.nan
    x[0, 3, 127] = -np.inf
    q = O.quantize_ex(x, "f32", O.E4M3, O.FLOOR, O.BOTH, block=O.BLOCK_32X32)
    s = q["row_scales"][0]
    assert s[1, 2] == 0xFF and s[0, 3] == 0xFF
    assert (s == 0xFF).sum() == 2
    assert (q["row_codes"][0, 32:64, 64:96] == 0x7F).all()
    assert q["col_scales"][0, 2, 1] == 0xFF


def test_2d_dequant_matches_1d_dequant_of_broadcast_scales():
    x = tiles_input(10)
    for fmt in (O.E2M1, O.E3M2, O.E4M3):
        q = O.quantize_ex(x, "f32", fmt, O.FLOOR, O.ROW, block=O.BLOCK_32X32)
        s1 = np.repeat(q["row_scales"], 32, axis=1)                           # [b, r, c/32]
        for out in ("f32", "bf16"):
            assert np.array_equal(O.dequantize_2d(q["row_codes"], q["row_scales"], fmt, out),
                                  O.dequantize(q["row_codes"], s1, fmt, out))
