"""Pins of the oracle's element encoder (round-to-nearest-even with saturation).

Independent references: a brute-force nearest-code scan over every code of the
format (written differently from the oracle's sorted-table search), torch's
float32 -> float8 casts (RNE; clamping to +-max first makes them saturate),
and exhaustive enumeration of every BF16 pattern under every shared scale.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O

FMTS = [O.E4M3, O.E5M2, O.E2M1, O.E2M3, O.E3M2]   # sign-magnitude formats


def brute_code(s: float, fmt) -> int:
    """Nearest code by scanning every code with the sign of s; ties -> even code."""
    sign = 1 if math.copysign(1.0, s) < 0 else 0
    best, best_d = None, None
    for c in range(1 << (fmt.bits - 1)):
        code = c | (sign << (fmt.bits - 1))
        v = O.decode_code(fmt, code)
        if math.isnan(v) or math.isinf(v):
            continue
        d = abs(abs(v) - abs(s))
        if best is None or d < best_d or (d == best_d and code % 2 == 0):
            best, best_d = code, d
    return best


def grid_probes(fmt):
    """Every code value, every midpoint, and one float64 step either side of each."""
    vals = sorted(set(abs(O.decode_code(fmt, c)) for c in range(1 << (fmt.bits - 1))
                      if math.isfinite(O.decode_code(fmt, c))))
    pts = list(vals) + [(a + b) / 2 for a, b in zip(vals[:-1], vals[1:])]
    pts += [vals[-1] * f for f in (1.01, 1.0625, 1.07, 1.5, 2.0, 1e6)]
    out = []
    for p in pts:
        out += [p, math.nextafter(p, math.inf), math.nextafter(p, 0.0)]
    out = [v for v in out if v >= 0.0]
    return out + [-v for v in out] + [0.0, -0.0]


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_encoder_matches_brute_force_scan(fmt):
    probes = grid_probes(fmt)
    got = O.encode_elements(np.array(probes), fmt)
    exp = [brute_code(s, fmt) for s in probes]
    assert got.tolist() == exp


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_ties_go_to_even_codes(fmt):
    # "MXFP4 と NVFP4 は何が違うのか調べてみた" §2: conversion to FP4 is roundTiesToEven.
    t = O.value_table(fmt)
    pos = [c for c in range(1 << (fmt.bits - 1)) if np.isfinite(t[c])]
    for a, b in zip(pos[:-1], pos[1:]):
        mid = (t[a] + t[b]) / 2
        code = int(O.encode_elements(np.array([mid]), fmt)[0])
        assert code == (a if a % 2 == 0 else b)
        assert code % 2 == 0


def test_saturation_boundaries():
    # E4M3 max 448 (§3 of the same article); values above clip (§4) rather than
    # becoming NaN (the saturate-or-NaN divergence named in §8).
    enc = lambda v, f: int(O.encode_elements(np.array([v]), f)[0])
    assert enc(448.0, O.E4M3) == 0x7E
    assert enc(464.0, O.E4M3) == 0x7E         # tie between 448 and 480 -> 448 (even)
    assert enc(480.0, O.E4M3) == 0x7E
    assert enc(1e9, O.E4M3) == 0x7E
    assert enc(-1e9, O.E4M3) == 0xFE
    assert enc(61440.0, O.E5M2) == 0x7B
    assert enc(1e30, O.E5M2) == 0x7B
    assert enc(7.0, O.E2M1) == 0x7
    assert enc(-100.0, O.E2M1) == 0xF
    assert enc(-0.0, O.E4M3) == 0x80
    assert enc(-0.0, O.E2M1) == 0x8


def _all_bf16_finite():
    bits = np.arange(1 << 16, dtype=np.uint32)
    mag = bits & 0x7FFF
    bits = bits[mag < 0x7F80]
    return (bits << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("fmt,tdt", [(O.E4M3, torch.float8_e4m3fn), (O.E5M2, torch.float8_e5m2)],
                         ids=["e4m3", "e5m2"])
def test_fp8_encoder_exhaustive_vs_torch(fmt, tdt):
    """Every finite BF16 pattern divided by every E8M0 scale 2^e: the oracle's
    code equals torch's RNE cast of the value clamped to +-max."""
    x = _all_bf16_finite()
    vmax = O.max_finite(fmt)
    for e in range(-127, 128):
        s = np.ldexp(x, -e)
        ours = O.encode_elements(s, fmt)
        clamped = np.clip(s, -vmax, vmax).astype(np.float32)       # exact where it matters
        ref = torch.from_numpy(clamped).to(tdt).view(torch.uint8).numpy()
        bad = np.nonzero(ours != ref)[0]
        assert bad.size == 0, (e, s[bad[:5]], ours[bad[:5]], ref[bad[:5]])


def test_e2m1_encoder_exhaustive_vs_brute_force():
    """Every finite BF16 pattern under every scale 2^e: vectorized brute force
    (distance to each of the 8 same-sign values, ties to the even code)."""
    x = _all_bf16_finite()
    t = O.value_table(O.E2M1)[:8]                     # 0 .. 6, codes 0..7
    for e in range(-127, 128):
        s = np.ldexp(x, -e)
        a = np.minimum(np.abs(s), 6.0)                # clip first so distances stay exact
        d = np.abs(a[:, None] - t[None, :])           # [n, 8]
        dmin = d.min(axis=1, keepdims=True)
        cand = d == dmin
        # among the nearest codes prefer the even one (at most two are nearest)
        even = cand & (np.arange(8)[None, :] % 2 == 0)
        mag = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
        ref = (mag | (np.signbit(s).astype(np.int64) << 3)).astype(np.uint8)
        ours = O.encode_elements(s, O.E2M1)
        assert np.array_equal(ours, ref), e
