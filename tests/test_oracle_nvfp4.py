"""Pins of the oracle's NVFP4 cast ("MXFP4 と NVFP4 は何が違うのか調べてみた" §3, §4
table and §7).

Independent references:
  * the page's formulas and sizes (16-element blocks, 72 bits per block, the
    global scale = tensor amax / (6 * 448), an unsigned block scale, E2M1's
    value table, decoding as an FP8 multiply then an FP32 multiply);
  * brute force in exact rationals (fractions.Fraction): the nearest grid
    value is the argmin of |q - v| over every value of the grid, ties to the
    even code, and FP32 / BF16 rounding is the nearest of the neighbouring
    floats. The E4M3 grid comes from torch's float8_e4m3fn decoder, the E2M1
    grid from the page's table;
  * closed forms for tensors built around a known amax, and error bounds.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

# [Q] §1 table: the 8 non-negative E2M1 values, codes 0..7
E2M1_VALUES = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4),
               Fraction(6)]
# UE4M3: the non-negative finite E4M3 codes 0x00..0x7E, decoded by torch
UE4M3_VALUES = [Fraction(float(v)) for v in
                torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).tolist()]


def nearest_code(q: Fraction, values) -> int:
    """Index of the value nearest to q, ties to the even index; the largest
    value for anything beyond it (argmin over the whole grid)."""
    best = None
    for code, v in enumerate(values):
        key = (abs(q - v), code % 2)
        if best is None or key < best[0]:
            best = (key, code)
    return best[1]


def round_to_float(q: Fraction, dt) -> float:
    """q rounded to nearest-even in numpy float dtype dt, by comparing the
    neighbours of a first guess exactly."""
    if q == 0:
        return 0.0
    sign = -1 if q < 0 else 1
    a = abs(q)
    top = Fraction(float(np.finfo(dt).max))
    if a >= top + (Fraction(2) ** 128 - top) / 2:               # IEEE: at or past max + half an ulp -> Inf
        return sign * float("inf")
    f = dt(min(float(a), float(top)))
    cands = [f, np.nextafter(f, dt(0)), np.nextafter(f, dt(np.inf))]
    cands = [c for c in cands if np.isfinite(c)]
    uint = np.uint32 if dt == np.float32 else np.uint16

    def key(c):
        return (abs(Fraction(float(c)) - a), int(np.array(c, dt).view(uint)) & 1)
    return sign * float(min(cands, key=key))


def brute_block(xs, g):
    """(UE4M3 code, E2M1 codes) of one finite 16-element block under global
    scale g (a finite positive FP32), in exact rationals."""
    gf = Fraction(float(g))
    amax = max(abs(Fraction(float(v))) for v in xs)
    s = nearest_code(amax / (6 * gf), UE4M3_VALUES)
    if s == 0:
        return s, [0] * len(xs)
    d = UE4M3_VALUES[s] * gf
    codes = []
    for v in xs:
        fv = Fraction(float(v))
        mag = nearest_code(abs(fv) / d, E2M1_VALUES)
        codes.append(mag | (8 if np.signbit(v) else 0))
    return s, codes


def rand(shape, seed, lo=-8, hi=8):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape) * np.exp2(rng.integers(lo, hi, size=shape[:-1] + (1,)))
    return x.astype(np.float32)


def f32_neighbours(v: float, k: int):
    """v (an FP32 value) and its k FP32 neighbours on each side, non-negative and finite."""
    out = [np.float32(v)]
    lo = hi = np.float32(v)
    for _ in range(k):
        lo = np.nextafter(lo, np.float32(0))
        hi = np.nextafter(hi, np.float32(np.inf))
        out += [lo, hi]
    return [o for o in out if np.isfinite(o) and o >= 0]


# global scales of the pins: ordinary, power of two, a 24-bit significand, FP32
# subnormal and near the top of FP32
G_PINS = [np.float32(1.0), np.float32(2.0 ** -10), np.float32(1.0) / np.float32(3.0), np.float32(0.0123),
          np.float32(1234.5678) / np.float32(2688.0), np.float32(2.0 ** -140), np.float32(3 * 2.0 ** -147),
          np.float32(1e30)]


def test_bits_per_element_and_block_size():
    # §3 table: 16 elements per block, 16 * 4 + 8 = 72 bits per block, 4.5 bits per element
    x = rand((1, 32, 64), 0)
    q = O.nvfp4_quantize(x, "f32", O.BOTH)
    n = x.size
    assert q["row_codes"].size == n // 2 and q["row_scales"].size == n // 16
    assert (q["row_codes"].size + q["row_scales"].size) * 8 / n == 4.5
    assert q["row_scales"].shape == (1, 32, 4) and q["col_scales"].shape == (1, 64, 2)
    assert q["global_scale"].dtype == np.float32 and q["global_scale"].shape == (1,)


def test_global_scale_is_amax_over_6_times_448():
    """§3: the FP32 global scale is the tensor's largest magnitude over 6 * 448,
    here the FP32 value nearest to the exact quotient."""
    rng = np.random.default_rng(11)
    amaxes = [2688.0, 2688.0 * 2 ** -10, 1.0, 3.3e38, 1e-30, 123.456, 2.0 ** -149, 5 * 2.0 ** -149, 2.0 ** -126]
    amaxes += list((rng.random(200) * np.exp2(rng.integers(-149, 127, 200))).astype(np.float32))
    for a in amaxes:
        a = np.float32(a)
        if a == 0 or not np.isfinite(a):
            continue
        x = np.zeros((1, 16, 32), np.float32)
        x[0, 3, 7] = -a
        x[0, 5, 9] = a / np.float32(3)
        g = O.nvfp4_quantize(x, "f32", O.ROW)["global_scale"][0]
        assert g == round_to_float(Fraction(float(a)) / 2688, np.float32), a
    assert O.nvfp4_quantize(np.full((1, 16, 16), 2688.0, np.float32), "f32", O.ROW)["global_scale"][0] == 1.0


def test_block_scale_brute_force_at_every_ue4m3_value_and_midpoint():
    """The block code is the UE4M3 value nearest to amax / (6 g): block maxima
    within 2 FP32 ulps of 6 g v for every UE4M3 value v and of 6 g m for every
    midpoint m between neighbouring values, under eight global scales."""
    pts = list(UE4M3_VALUES[1:]) + [(a + b) / 2 for a, b in zip(UE4M3_VALUES[:-1], UE4M3_VALUES[1:])]
    pts += [Fraction(464), Fraction(480), Fraction(10 ** 6)]           # beyond 448: saturation
    for g in G_PINS:
        gf = Fraction(float(g))
        amax = []
        for p in pts:
            t = round_to_float(6 * gf * p, np.float32)
            if np.isfinite(t):
                amax += f32_neighbours(t, 2)
        amax = np.array(amax, np.float32)
        got = O.ue4m3_encode(amax.astype(np.float64), np.full(amax.shape, g))
        exp = np.array([nearest_code(Fraction(float(a)) / (6 * gf), UE4M3_VALUES) for a in amax])
        bad = np.nonzero(got != exp)[0]
        assert bad.size == 0, (g, amax[bad[:3]], got[bad[:3]], exp[bad[:3]])


@pytest.mark.parametrize("g", G_PINS[:6])
def test_element_codes_brute_force_under_every_block_scale(g):
    """Whole blocks through nvfp4_quantize with a given g: for every UE4M3
    block code, a block max that selects it and elements within 1 FP32 ulp of
    every E2M1 value and every midpoint (times s g), both signs."""
    gf = Fraction(float(g))
    e2 = list(E2M1_VALUES[1:]) + [(a + b) / 2 for a, b in zip(E2M1_VALUES[:-1], E2M1_VALUES[1:])]
    blocks = []
    for s in range(1, 0x7F):
        top = round_to_float(6 * gf * UE4M3_VALUES[s], np.float32)
        if not np.isfinite(top) or top == 0:
            continue
        vals = []
        for p in e2:
            vals += f32_neighbours(round_to_float(p * UE4M3_VALUES[s] * gf, np.float32), 1)
        vals = [v for v in vals if v <= top]
        for i in range(0, len(vals), 15):
            chunk = vals[i:i + 15]
            blk = [np.float32(top)] + [np.float32(-v) if (j % 3 == 1) else np.float32(v) for j, v in enumerate(chunk)]
            blk += [np.float32(0.0)] * (16 - len(blk))
            blocks.append(blk)
    x = np.array(blocks, np.float32).reshape(1, -1, 16)
    q = O.nvfp4_quantize(x, "f32", O.ROW, global_scale=np.array([g], np.float32))
    codes = O.unpack_e2m1(q["row_codes"])[0]
    for i, blk in enumerate(blocks):
        s, c = brute_block(blk, g)
        assert q["row_scales"][0, i, 0] == s, (g, i, blk[0])
        assert list(codes[i]) == c, (g, i, [float(v) for v in blk], list(codes[i]), c)


def test_midpoint_ties_go_to_even_codes():
    """A = 2688 makes g = 1, and a block max of 18 makes the block scale 3
    (0x44), so x / 3 is exact: 0.75 -> 0.25 (between 0 and 0.5) -> 0;
    2.25 -> 0.75 -> 1.0; 7.5 -> 2.5 -> 2.0; 15 -> 5 -> 4.0; 4.5 -> 1.5 (a
    value) -> 1.5. A multiply by fp32(1 / 3) would see these quotients off
    their midpoints."""
    x = np.zeros((1, 2, 16), np.float32)
    x[0, 0, 0] = 2688.0
    x[0, 1, :6] = [18.0, 0.75, -0.75, 2.25, 7.5, 15.0]
    x[0, 1, 6] = 4.5
    q = O.nvfp4_quantize(x, "f32", O.ROW)
    assert q["global_scale"][0] == 1.0
    assert q["row_scales"][0, 1, 0] == 0x44
    c = O.unpack_e2m1(q["row_codes"])[0, 1]
    assert list(c[:7]) == [0x7, 0x0, 0x8, 0x2, 0x4, 0x6, 0x3]


def test_block_holding_the_tensor_max_decodes_exactly():
    """With A = 2688 * 2^k the global scale is exactly 2^k; the block holding A
    gets scale 448 (code 0x7E) and A itself code 6 (0x7), so it decodes to A."""
    for k in (-20, 0, 7):
        x = rand((1, 64, 64), 1, -4, 0) * np.float32(2.0 ** k)
        A = np.float32(2688.0 * 2.0 ** k)
        x[0, 10, 17] = A
        q = O.nvfp4_quantize(x, "f32", O.ROW)
        assert q["global_scale"][0] == np.float32(2.0 ** k)
        assert q["row_scales"][0, 10, 1] == 0x7E
        codes = O.unpack_e2m1(q["row_codes"])[0]
        assert codes[10, 17] == 0x7
        y = O.nvfp4_dequantize(q["row_codes"], q["row_scales"], q["global_scale"], "f32").view(np.float32)
        assert y[0, 10, 17] == A


def test_block_scales_are_unsigned_e4m3():
    # §3 / §7: the block scale is an unsigned E4M3: no code carries the sign bit
    x = rand((2, 64, 128), 2, -30, 30)
    q = O.nvfp4_quantize(x, "f32", O.BOTH)
    for k in ("row_scales", "col_scales"):
        assert (q[k] < 0x80).all()
        assert (q[k] != 0x7F).all()                               # no NaN without NaN input


def test_random_blocks_brute_force():
    """Random FP32 and BF16 tensors, every block against the brute force."""
    x = rand((1, 8, 64), 3, -12, 12)
    xb = torch.from_numpy(rand((1, 8, 64), 9, -6, 6)).bfloat16()
    for arr, dt in ((x, "f32"), (xb.view(torch.int16).numpy().view(np.uint16), "bf16")):
        q = O.nvfp4_quantize(arr, dt, O.ROW)
        vals = O.widen(arr, dt).astype(np.float32)[0]
        g = q["global_scale"][0]
        assert g == round_to_float(Fraction(float(np.abs(vals).max())) / 2688, np.float32)
        codes = O.unpack_e2m1(q["row_codes"])[0]
        for r in range(vals.shape[0]):
            for b in range(vals.shape[1] // 16):
                s, c = brute_block(vals[r, 16 * b:16 * b + 16], g)
                assert q["row_scales"][0, r, b] == s
                assert list(codes[r, 16 * b:16 * b + 16]) == c


@pytest.mark.parametrize("seed", [4, 5])
def test_round_trip_error_bound(seed):
    """Every element decodes within half an E2M1 step (times the block's
    decoded scale) of x, or within the clip of the block max (UE4M3 rounding
    can leave the largest element of a block up to 1/16 above 6 * s * g)."""
    x = rand((1, 256, 128), seed, -20, 20)
    q = O.nvfp4_quantize(x, "f32", O.ROW)
    y = O.nvfp4_dequantize(q["row_codes"], q["row_scales"], q["global_scale"], "f32").view(np.float32)
    g = np.float64(q["global_scale"][0])
    sg = O.value_table(O.E4M3)[q["row_scales"][0].astype(int)].repeat(16, axis=1) * g
    a = np.abs(x[0].astype(np.float64))
    err = np.abs(y[0].astype(np.float64) - x[0])
    ok_scale = sg > 0
    half_step = np.where(a / np.where(ok_scale, sg, 1) < 2, 0.25, np.where(a / np.where(ok_scale, sg, 1) < 4, 0.5, 1.0))
    within = err <= half_step * sg * (1 + 2 ** -20) + 1e-45
    clipped = ok_scale & (a > 6 * sg)
    assert np.all(within | clipped | ~ok_scale)
    # blocks whose scale is below UE4M3's range (relative to the tensor max) decode to 0
    assert np.all(y[0][~ok_scale] == 0)
    # the clipped ones decode to 6 * s * g (rounded once to FP32)
    assert np.all(np.abs(err[clipped] - (a[clipped] - 6 * sg[clipped])) <= 6 * sg[clipped] * 2.0 ** -23)
    # and the scale was rounded down by at most half a UE4M3 step (1/16 relative for
    # normal scales, 2^-10 absolute for subnormal ones): a <= 6 * (s + step/2) * g
    sv = O.value_table(O.E4M3)[q["row_scales"][0].astype(int)].repeat(16, axis=1)
    half = np.where(sv >= 2.0 ** -6, sv / 16, 2.0 ** -10)
    assert np.all(a[clipped] <= 6 * (sv[clipped] + half[clipped]) * g * (1 + 2 ** -20))


def test_zero_tensor_special_blocks_and_unusable_global_scales():
    z = np.zeros((1, 16, 32), np.float32)
    q = O.nvfp4_quantize(z, "f32", O.BOTH)
    assert q["global_scale"][0] == 0.0
    assert (q["row_scales"] == 0).all() and (q["row_codes"] == 0).all()
    x = rand((1, 32, 64), 6)
    x[0, 5, 20] = np.nan
    x[0, 30, 3] = -np.inf
    q = O.nvfp4_quantize(x, "f32", O.ROW)
    fin = np.abs(np.where(np.isfinite(x), x, 0)).max()
    assert q["global_scale"][0] == np.float32(fin) / np.float32(2688)   # non-finite ignored
    s = q["row_scales"][0]
    assert s[5, 1] == 0x7F and s[30, 0] == 0x7F and (s == 0x7F).sum() == 2
    y = O.nvfp4_dequantize(q["row_codes"], q["row_scales"], q["global_scale"], "f32")[0]
    assert (y[5, 16:32] == 0x7FC00000).all() and (y[30, 0:16] == 0x7FC00000).all()
    assert not (y[0] == 0x7FC00000).any()
    # a given g that is 0, negative, infinite or NaN: finite blocks store scale 0 and codes 0
    for g in (0.0, -1.0, np.inf, np.nan):
        q = O.nvfp4_quantize(x, "f32", O.ROW, global_scale=np.array([g], np.float32))
        fin_blocks = q["row_scales"][0] != 0x7F
        assert (q["row_scales"][0][fin_blocks] == 0).all() and (q["row_codes"] == 0).all()
        assert (q["row_scales"][0] == 0x7F).sum() == 2


def test_column_copy_shares_the_global_scale():
    x = rand((2, 64, 96), 7)
    q = O.nvfp4_quantize(x, "f32", O.BOTH)
    t = O.nvfp4_quantize(np.ascontiguousarray(x.transpose(0, 2, 1)), "f32", O.ROW)
    assert np.array_equal(q["global_scale"], t["global_scale"])
    assert np.array_equal(q["col_codes"], t["row_codes"])
    assert np.array_equal(q["col_scales"], t["row_scales"])
    # and each batch slice has its own global scale: scaling slice 1 by 8 scales
    # only its global scale, by 8 (exactly: 8 is a power of two), and keeps its codes
    x[1] *= 8
    q2 = O.nvfp4_quantize(x, "f32", O.ROW)
    assert q2["global_scale"][0] == q["global_scale"][0]
    assert q2["global_scale"][1] == q["global_scale"][1] * 8
    assert np.array_equal(q2["row_codes"], q["row_codes"]) and np.array_equal(q2["row_scales"], q["row_scales"])


@pytest.mark.parametrize("g", [np.float32(1.7e-3), np.float32(2.0 ** -140), np.float32(3e35)])
def test_dequant_every_code_under_every_scale(g):
    """§4 table: decoding is an FP8 multiply, then an FP32 multiply by g. Every
    E2M1 code under every UE4M3 code, against the exact product rounded once
    to FP32 (and that FP32 value rounded to BF16)."""
    scales = np.arange(0, 0x80, dtype=np.uint8).reshape(1, -1, 1)          # 0x7F: NaN
    nib = np.tile(np.arange(16, dtype=np.uint8), 1)
    codes = np.broadcast_to((nib[0::2] | (nib[1::2] << 4)), (1, 128, 8)).copy()
    y = O.nvfp4_dequantize(codes, scales, np.array([g], np.float32), "f32").view(np.float32)[0]
    yb = O.nvfp4_dequantize(codes, scales, np.array([g], np.float32), "bf16")[0]
    e2 = [E2M1_VALUES[c & 7] * (-1 if c & 8 else 1) for c in range(16)]
    for s in range(128):
        for c in range(16):
            if s == 0x7F:
                assert np.isnan(y[s, c]) and yb[s, c] == 0x7FC0
                continue
            ref = round_to_float(e2[c] * UE4M3_VALUES[s] * Fraction(float(g)), np.float32)
            assert y[s, c] == ref or (y[s, c] == 0 and ref == 0), (s, c)
            refb = torch.tensor(np.float32(ref)).bfloat16().view(torch.int16).item() & 0xFFFF
            assert yb[s, c] == refb or (ref == 0 and yb[s, c] & 0x7FFF == 0), (s, c)
