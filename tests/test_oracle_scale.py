"""Pins of the oracle's shared-exponent (E8M0 scale) rules.

References: brute-force searches over every E8M0 exponent written straight from
each rule's definition (in float64 and in exact rationals), the landing
intervals the pages print, and the special cases (zero, NaN/Inf blocks, the
clamp at 2^-127).
"""
import math

import numpy as np
import pytest
import torch

import oracle as O

FMTS = [O.E4M3, O.E5M2, O.E2M1, O.E2M3, O.E3M2, O.INT8]


def brute_floor(amax: float, fmt) -> int:
    """Largest e in [-127, 127] with 2^(e + emax) <= amax; -127 if none (incl. amax = 0)."""
    em = O.emax_of(fmt)
    best = -127
    for e in range(-127, 128):
        if math.ldexp(1.0, e + em) <= amax:
            best = e
    return best


def brute_roundup(amax: float, fmt) -> int:
    """Smallest e in [-127, 127] with amax <= max * 2^e."""
    vmax = O.max_finite(fmt)
    for e in range(-127, 128):
        if amax <= math.ldexp(vmax, e):
            return e
    return 127


def amax_samples():
    bf = np.arange(0, 0x7F80, dtype=np.uint32) << 16                  # every finite BF16 magnitude
    v = list(bf.view(np.float32).astype(np.float64))
    rng = np.random.default_rng(7)
    f32 = rng.integers(0, 0x7F800000, size=4000, dtype=np.uint32).view(np.float32)
    v += list(f32.astype(np.float64))
    v += [float(np.float32(2.0 ** -149)), 2.0 ** -126, 1.75 * 2.0 ** -119,
          float(np.nextafter(np.float32(1.75 * 2.0 ** -119), np.float32(1))), 6 * 2.0 ** -127,
          float(np.finfo(np.float32).max)]
    return np.array(v)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_floor_rule_matches_brute_force(fmt):
    a = amax_samples()
    ours = O.shared_exponent(a, fmt, O.FLOOR)
    idx = np.linspace(0, len(a) - 1, 6000).astype(int)
    for i in idx:
        assert ours[i] == brute_floor(a[i], fmt), a[i]


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_roundup_rule_matches_brute_force(fmt):
    a = amax_samples()
    ours = O.shared_exponent(a, fmt, O.ROUNDUP)
    idx = np.linspace(0, len(a) - 1, 6000).astype(int)
    for i in idx:
        assert ours[i] == brute_roundup(a[i], fmt), a[i]


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_landing_intervals(fmt):
    # "MXFP4 と NVFP4 は何が違うのか調べてみた" §4: the floor rule lands the scaled
    # block max in [4, 8) for E2M1 (generally [2^emax, 2^(emax+1))); the round-up
    # rule lands it in (3, 6] (generally (max/2, max]).
    a = amax_samples()
    a = a[a > 0]
    em, vmax = O.emax_of(fmt), O.max_finite(fmt)
    ef = O.shared_exponent(a, fmt, O.FLOOR)
    s = np.ldexp(a, -ef)
    free = ef > -127
    assert ((s[free] >= 2.0 ** em) & (s[free] < 2.0 ** (em + 1))).all()
    eu = O.shared_exponent(a, fmt, O.ROUNDUP)
    s = np.ldexp(a, -eu)
    # INT8 (emax 0) can need e = 128 for block maxima above 127/64 * 2^127; the
    # clamp at 127 then clips them, as it does under the floor rule
    free = (eu > -127) & (eu < 127)
    assert ((s[free] > vmax / 2) & (s[free] <= vmax)).all()
    assert (s[eu == -127] <= vmax).all()
    top = eu == 127
    assert (np.ldexp(a[top], -127) <= vmax).all() or fmt.integer
    # the two rules differ by at most one step, and only when the floor rule would clip
    d = eu - ef
    assert set(np.unique(d).tolist()) <= {0, 1}
    assert (np.ldexp(a[d == 1], -ef[d == 1]) > vmax).all()


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_roundup_matches_exact_rational_search(fmt):
    """The smallest e with amax <= max * 2^e, found with exact rational arithmetic
    (fractions.Fraction) by stepping from the floor exponent."""
    from fractions import Fraction
    a = amax_samples()
    a = a[a > 0]
    vmax = Fraction(O.max_finite(fmt))
    ours = O.shared_exponent(a, fmt, O.ROUNDUP)
    for v, e in zip(a[::7], ours[::7]):
        fv = Fraction(float(v))
        k = -127
        while k < 127 and fv > vmax * Fraction(2) ** k:
            k += 1
        assert e == k, v


def test_roundup_edge_below_fp32_normal_quotient():
    # amax just above 1.75 * 2^-119 with E4M3: the exact rule needs e = -126
    # (448 * 2^-127 is below amax); a quotient amax/448 formed in FP32 would be
    # subnormal and round to 2^-127.
    amax = float(np.nextafter(np.float32(1.75 * 2.0 ** -119), np.float32(1.0)))
    assert O.shared_exponent(np.array([amax]), O.E4M3, O.ROUNDUP)[0] == -126
    assert brute_roundup(amax, O.E4M3) == -126
    assert O.shared_exponent(np.array([1.75 * 2.0 ** -119]), O.E4M3, O.ROUNDUP)[0] == -127


def test_special_and_zero_blocks():
    # §2: 0xFF is NaN and there is no Inf, so a block holding NaN or Inf takes
    # scale 0xFF; an all-zero block takes the smallest scale, code 0x00.
    blocks = np.zeros((5, 32))
    blocks[1, 3] = np.nan
    blocks[2, 31] = -np.inf
    blocks[3, 0] = np.inf
    blocks[3, 1] = np.nan
    blocks[4, :] = -0.0
    for fmt in FMTS:
        for mode in (O.FLOOR, O.ROUNDUP):
            codes, scales = O.quantize_blocks(blocks, fmt, mode)
            assert scales.tolist() == [0, 255, 255, 255, 0]
            # FP8 has a NaN code (S.1111.111 / S.11111.11); the others have none
            fill = {"e4m3": 0x7F, "e5m2": 0x7F}.get(fmt.name, 0x0)
            assert (codes[1:4] == fill).all()
            assert (codes[0] == 0).all()
            # -0 keeps its sign bit; two's-complement INT8 has no negative zero
            neg_zero = {"e4m3": 0x80, "e5m2": 0x80, "e2m1": 0x8, "e2m3": 0x20, "e3m2": 0x20, "int8": 0x0}
            assert (codes[4] == neg_zero[fmt.name]).all()


def test_scale_clamp_and_subnormal_inputs():
    # A block whose floor exponent would fall below -127 is clamped to 2^-127;
    # its FP32-subnormal elements are then scaled up into the format's range.
    blk = np.zeros((1, 32))
    blk[0, 0] = 2.0 ** -140
    blk[0, 1] = -(2.0 ** -149)
    codes, scales = O.quantize_blocks(blk, O.E5M2, O.FLOOR)
    assert scales[0] == 0
    # 2^-140 * 2^127 = 2^-13 -> E5M2 normal, exponent field -13 + 15 = 2
    assert codes[0, 0] == (2 << 2)
    # 2^-149 * 2^127 = 2^-22 is below half the E5M2 minimum 2^-16 -> -0
    assert codes[0, 1] == 0x80
