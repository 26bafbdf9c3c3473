"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in the oracle (on the CPU, for the duration of the
test) and checks that at least one of the pin tests then fails. A pin suite
that still passed with the mistake in place would not be pinning that part of
the oracle.
"""
import contextlib

import numpy as np
import pytest

import oracle as O
import oracle.mx_oracle as M
import test_oracle_dequant as PD
import test_oracle_encode as PE
import test_oracle_formats as PF
import test_oracle_fp6_int8 as P6
import test_oracle_invariants as PI
import test_oracle_scale as PS
import test_oracle_worked_example as PW


@contextlib.contextmanager
def planted(name, fn):
    """Replace oracle function `name` in the module and the package namespace."""
    old = getattr(M, name)
    setattr(M, name, fn)
    setattr(O, name, fn)
    try:
        yield
    finally:
        setattr(M, name, old)
        setattr(O, name, old)


def fails(check, *args):
    try:
        check(*args)
    except AssertionError:
        return True
    return False


def any_pin_fails(checks):
    return any(fails(c, *a) for c, a in checks)


# ---- planted mistakes ----

def enc_ties_away(s, fmt):
    """Round half away from zero instead of to even."""
    codes_pos, vals_pos = M.positive_grid(fmt)
    a = np.abs(s)
    idx = np.clip(np.searchsorted(vals_pos, a), 1, len(vals_pos) - 1)
    lo, hi = idx - 1, idx
    pick_hi = (vals_pos[hi] - a) <= (a - vals_pos[lo])
    mag = np.where(pick_hi, codes_pos[hi], codes_pos[lo])
    mag = np.where(a >= vals_pos[-1], codes_pos[-1], mag)
    return (mag | (np.signbit(s).astype(np.int64) << (fmt.bits - 1))).astype(np.uint8)


def enc_no_saturation(s, fmt):
    """Overflow becomes the NaN / all-ones code instead of +-max."""
    c = M._orig_encode(s, fmt)
    over = np.abs(s) > M.max_finite(fmt)
    return np.where(over, (c | 0x7F) if fmt.bits == 8 else c, c).astype(np.uint8)


def enc_unsigned_zero(s, fmt):
    """The sign of zero is dropped."""
    c = M._orig_encode(s, fmt)
    zero = (s == 0)
    return np.where(zero, 0, c).astype(np.uint8)


def shexp_emax_plus_one(amax, fmt, mode):
    """The floor rule subtracts emax + 1."""
    e = M._orig_shexp(amax, fmt, mode)
    return np.clip(np.where(amax > 0, e - 1, e), -127, 127)


def shexp_roundup_ge(amax, fmt, mode):
    """Round-up rule bumps also when amax equals max * 2^(E - emax) exactly."""
    amax = np.asarray(amax, dtype=np.float64)
    if mode != O.ROUNDUP:
        return M._orig_shexp(amax, fmt, mode)
    em, vmax = M.emax_of(fmt), M.max_finite(fmt)
    big_e = np.frexp(amax)[1].astype(np.int64) - 1
    e = big_e - em + (amax >= np.ldexp(vmax, big_e - em)).astype(np.int64)
    e = np.where(amax == 0, -127, e)
    return np.clip(e, -127, 127)


def quantize_untransposed(x, in_dtype, fmt, mode, axis):
    """The column plane keeps X's [B][R][C] element order instead of X^T's."""
    out = M._orig_quantize(x, in_dtype, fmt, mode, axis)
    if "col_codes" in out and fmt.bits == 8:
        cc = out["col_codes"]                                   # [B][C][R]
        out["col_codes"] = np.ascontiguousarray(cc.transpose(0, 2, 1)).reshape(cc.shape)
    return out


def pack_swapped(codes):
    c = np.asarray(codes, dtype=np.uint8)
    return ((c[..., 0::2] & 0xF) << 4) | (c[..., 1::2] & 0xF)


def dequant_bias_126(codes, scales, fmt, out_dtype):
    """The E8M0 bias is taken as 126: every scale code reads one step high."""
    shifted = np.minimum(np.asarray(scales, np.int64) + 1, 254).astype(np.uint8)
    return M._orig_dequant(codes, shifted, fmt, out_dtype)


def pack_fp6_msb_first(codes):
    """The 6-bit stream is built most significant bit first."""
    c = np.asarray(codes, dtype=np.uint8)
    bits = np.unpackbits(c[..., None], axis=-1)[..., 2:]
    return np.packbits(bits.reshape(c.shape[:-1] + (c.shape[-1] * 6,)), axis=-1)


def enc_int8_sign_magnitude(s, fmt):
    """INT8 negatives get a sign bit instead of two's complement."""
    c = M._orig_encode(s, fmt)
    if not fmt.integer:
        return c
    neg = np.signbit(s) & (c != 0)
    return np.where(neg, ((-c.astype(np.int64)) & 0x7F) | 0x80, c).astype(np.uint8)


def decode_e3m2_bias_4(fmt, code):
    """E3M2 read with bias 4 instead of 3."""
    v = M._orig_decode(fmt, code)
    return v / 2.0 if fmt.name == "e3m2" else v


@pytest.fixture(autouse=True)
def keep_originals():
    M._orig_encode = M.encode_elements
    M._orig_shexp = M.shared_exponent
    M._orig_quantize = M.quantize
    M._orig_dequant = M.dequantize
    M._orig_decode = M.decode_code
    yield


def test_pins_catch_ties_away_from_zero():
    with planted("encode_elements", enc_ties_away):
        assert any_pin_fails([(PE.test_ties_go_to_even_codes, (O.E2M1,)),
                              (PE.test_encoder_matches_brute_force_scan, (O.E4M3,))])


def test_pins_catch_missing_saturation():
    with planted("encode_elements", enc_no_saturation):
        assert any_pin_fails([(PE.test_saturation_boundaries, ())])


def test_pins_catch_unsigned_zero():
    with planted("encode_elements", enc_unsigned_zero):
        assert any_pin_fails([(PE.test_saturation_boundaries, ()),
                              (PS.test_special_and_zero_blocks, ())])


def test_pins_catch_emax_off_by_one():
    with planted("shared_exponent", shexp_emax_plus_one):
        assert any_pin_fails([(PS.test_floor_rule_matches_brute_force, (O.E2M1,)),
                              (PW.test_shared_scale_is_2_pow_minus_4_under_both_rules, ())])


def test_pins_catch_roundup_boundary():
    with planted("shared_exponent", shexp_roundup_ge):
        assert any_pin_fails([(PS.test_roundup_rule_matches_brute_force, (O.E4M3,)),
                              (PS.test_landing_intervals, (O.E4M3,))])


def test_pins_catch_untransposed_column_plane():
    with planted("quantize", quantize_untransposed):
        assert any_pin_fails([(PI.test_column_copy_orientation_closed_form, (O.E4M3,))])


def test_pins_catch_swapped_nibbles():
    with planted("pack_e2m1", pack_swapped):
        assert any_pin_fails([(PI.test_e2m1_nibble_order, ()),
                              (PW.test_scaled_values_printed_on_the_page, ())])


def test_pins_catch_scale_bias_off_by_one():
    with planted("dequantize", dequant_bias_126):
        assert any_pin_fails([(PF.test_e8m0_range_and_nan_scale, ()),
                              (PD.test_overflow_at_top_of_range_is_inf, ())])


def test_pins_catch_fp6_bit_order():
    with planted("pack_fp6", pack_fp6_msb_first):
        assert any_pin_fails([(P6.test_fp6_packing_closed_form, ())])


def test_pins_catch_int8_sign_magnitude():
    with planted("encode_elements", enc_int8_sign_magnitude):
        assert any_pin_fails([(P6.test_int8_encoder_exhaustive_vs_numpy_rint, ()),
                              (P6.test_int8_encoder_matches_brute_force_scan, ())])


def test_pins_catch_e3m2_bias():
    with planted("decode_code", decode_e3m2_bias_4):
        assert any_pin_fails([(P6.test_fp6_tables_are_fp8_low_binades, ("e3m2",))])


# ---- stochastic rounding, random bits, 2-D blocks ----

import oracle.mx_variants as V  # noqa: E402
import test_oracle_variants as PV  # noqa: E402


@contextlib.contextmanager
def planted_v(name, fn):
    old = getattr(V, name)
    setattr(V, name, fn)
    setattr(O, name, fn)
    try:
        yield
    finally:
        setattr(V, name, old)
        setattr(O, name, old)


def test_pins_catch_philox_swapped_multipliers():
    orig = V.philox4x32_10

    def swapped(ctr, key):
        V._M0, V._M1 = V._M1, V._M0
        try:
            return orig(ctr, key)
        finally:
            V._M0, V._M1 = V._M1, V._M0
    with planted_v("philox4x32_10", swapped):
        assert any_pin_fails([(PV.test_philox_known_answers, KAT) for KAT in PV.KAT])


def test_pins_catch_sr_ge_comparison():
    def ge(s, fmt, u16):
        """f >= u instead of f > u: a draw of 0 then moves grid values up."""
        s = np.asarray(s, dtype=np.float64)
        a = np.abs(s)
        nz = a > 0
        q = V._spacing(np.where(nz, a, 1.0), fmt)
        x = a / q
        n = np.floor(x)
        up = (x - n) >= np.asarray(u16, dtype=np.float64) / 65536.0
        mag = np.where(a >= M.max_finite(fmt), M.max_finite(fmt), (n + up) * q)
        return M.encode_elements(np.copysign(np.where(nz, mag, 0.0), s), fmt)
    with planted_v("encode_elements_sr", ge):
        assert any_pin_fails([(PV.test_sr_leaves_grid_values_and_saturates, ()),
                              (PV.test_sr_up_count_over_all_draws, (O.E2M1,))])


def test_pins_catch_sr_bits_in_transposed_order():
    orig = V.quantize_ex

    def transposed_bits(x, in_dtype, fmt, mode, axis, rounding="rne", seed=0, block="1x32"):
        if rounding != "sr" or not (axis & O.COL):
            return orig(x, in_dtype, fmt, mode, axis, rounding, seed, block)
        # column copy drawn with X^T's own flat order
        xt = np.ascontiguousarray(np.swapaxes(np.asarray(x), -1, -2))
        out = orig(x, in_dtype, fmt, mode, axis & O.ROW, rounding, seed, block) if axis & O.ROW else {}
        t = orig(xt, in_dtype, fmt, mode, O.ROW, rounding, seed, block)
        out["col_codes"], out["col_scales"] = t["row_codes"], t["row_scales"]
        return out
    with planted_v("quantize_ex", transposed_bits):
        assert any_pin_fails([(PV.test_sr_column_copy_uses_the_elements_bits, ())])


def test_pins_catch_2d_scale_from_first_row():
    orig_plane = V._quant_plane

    def plane(x64, u, fmt, mode, block):
        """Each 32x32 tile takes the scale of its first row only."""
        if block != "32x32":
            return orig_plane(x64, u, fmt, mode, block)
        first = np.repeat(x64[:, ::32, :], 32, axis=1)
        _, scales_f = orig_plane(first, u, fmt, mode, block)
        codes, _ = orig_plane(x64, u, fmt, mode, block)
        return codes, scales_f
    with planted_v("_quant_plane", plane):
        assert any_pin_fails([(PV.test_2d_scale_is_max_of_row_block_scales, (O.E4M3, O.FLOOR))])


# ---- NVFP4 ----

import oracle.nvfp4 as NV  # noqa: E402
import test_oracle_nvfp4 as PN  # noqa: E402


@contextlib.contextmanager
def planted_nv(name, fn):
    old = getattr(NV, name)
    setattr(NV, name, fn)
    setattr(O, name, fn)
    try:
        yield
    finally:
        setattr(NV, name, old)
        setattr(O, name, old)


NV_PINS = [(PN.test_global_scale_is_amax_over_6_times_448, ()),
           (PN.test_block_scale_brute_force_at_every_ue4m3_value_and_midpoint, ()),
           (PN.test_element_codes_brute_force_under_every_block_scale, (np.float32(1.0) / np.float32(3.0),)),
           (PN.test_midpoint_ties_go_to_even_codes, ()), (PN.test_block_holding_the_tensor_max_decodes_exactly, ()),
           (PN.test_random_blocks_brute_force, ())]


def test_pins_catch_nvfp4_global_scale_without_the_6():
    def g448(x64):
        b = x64.shape[0]
        a = np.abs(np.where(np.isfinite(x64), x64, 0.0)).reshape(b, -1).max(axis=1)
        return a.astype(np.float32) / np.float32(448.0)
    with planted_nv("nvfp4_global_scale", g448):
        assert any_pin_fails(NV_PINS)


def test_pins_catch_nvfp4_elements_scaled_without_global():
    orig = NV._quant_plane

    def no_global(x64, g):
        return orig(x64, np.ones_like(g))
    with planted_nv("_quant_plane", no_global):
        assert any_pin_fails(NV_PINS)


def test_pins_catch_nvfp4_fp32_reciprocal_chain():
    """Every step in FP32: block code of fp32(fp32(amax / 6) / g), elements
    fp32(x * fp32(1 / fp32(s * g))), each then rounded to the grid."""
    def chain(x64, g):
        b, r, c = x64.shape
        blocks = x64.reshape(b, r, c // 16, 16)
        special = ~np.isfinite(blocks).all(axis=3)
        clean = np.where(np.isfinite(blocks), blocks, 0.0)
        amax = np.abs(clean).max(axis=3).astype(np.float32)
        gg = np.asarray(g, np.float32).reshape(b, 1, 1)
        with np.errstate(all="ignore"):
            t = (amax / np.float32(6)) / gg
            scode = M.encode_elements(np.minimum(t.astype(np.float64), 448.0), M.E4M3)
            rb = np.float32(1) / (M.value_table(M.E4M3)[scode].astype(np.float32) * gg)
            q = clean.astype(np.float32) * rb[..., None]
        zero = (scode == 0)[..., None] | special[..., None] | ~np.isfinite(rb)[..., None]
        codes = np.where(zero, 0, M.encode_elements(np.where(zero, 0.0, q.astype(np.float64)), M.E2M1))
        scode = np.where(special, 0x7F, scode).astype(np.uint8)
        return M.pack_e2m1(codes.astype(np.uint8).reshape(b, r, c)), scode
    with planted_nv("_quant_plane", chain):
        assert any_pin_fails(NV_PINS)


def test_pins_catch_nvfp4_block_scale_rounded_twice():
    def twice(amax, g):
        with np.errstate(all="ignore"):
            t = (np.asarray(amax, np.float32) / np.float32(6)) / np.asarray(g, np.float32)
        return M.encode_elements(np.minimum(t.astype(np.float64), 448.0), M.E4M3).astype(np.uint8)
    with planted_nv("ue4m3_encode", twice):
        assert any_pin_fails(NV_PINS)


def test_pins_catch_nvfp4_ties_away_from_zero():
    orig = NV.nearest_code_of_quotient

    def away(num, den, fmt):
        codes = orig(num, den, fmt)
        cs, vals = M.positive_grid(fmt)
        mids = (vals[:-1] + vals[1:]) / 2
        n, d = (a.reshape(-1) for a in np.broadcast_arrays(np.asarray(num, np.float64), np.asarray(den, np.float64)))
        for k, m in enumerate(mids):
            codes = np.where(n == m * d, cs[k + 1], codes)     # every tie goes up
        return codes
    with planted_nv("nearest_code_of_quotient", away):
        assert any_pin_fails(NV_PINS)


import oracle.nested as NS  # noqa: E402
import test_oracle_nested as PNS  # noqa: E402

NESTED_PINS = [(PNS.test_512_subtiles_per_block, ()), (PNS.test_lossless_below_threshold, (14,)),
               (PNS.test_spread_15_loses_exactly_the_predicted_elements, ()),
               (PNS.test_block_scale_places_the_largest_value_at_384, ()),
               (PNS.test_zero_and_nan_subblocks_do_not_count, ()), (PNS.test_ragged_blocks_and_transpose, ()),
               (PNS.test_pipeline_from_fp32_weights, ())]


@contextlib.contextmanager
def planted_nested(name, value):
    old = getattr(NS, name)
    setattr(NS, name, value)
    try:
        yield
    finally:
        setattr(NS, name, old)


@pytest.mark.parametrize("shift", [5, 7])
def test_pins_catch_nested_block_scale_off_by_one(shift):
    with planted_nested("SHIFT", shift):
        assert any_pin_fails(NESTED_PINS)


def test_pins_catch_nested_zero_subblocks_counted():
    with planted_nested("_active", lambda qs, k: k != M.E8M0_NAN):
        assert any_pin_fails(NESTED_PINS)


def test_pins_catch_nested_nan_subblocks_counted():
    with planted_nested("_active", lambda qs, k: ((qs & 0x7) != 0).any(axis=-1)):
        assert any_pin_fails(NESTED_PINS)


def test_pins_catch_nested_64_blocks():
    with planted_nested("FP8_BLOCK", 64):
        assert any_pin_fails(NESTED_PINS)
