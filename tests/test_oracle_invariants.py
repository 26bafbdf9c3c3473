"""Invariants of the quantize / dequantize pair and layout pins of the oracle."""
import numpy as np
import pytest

import mx_inputs as I
import oracle as O

FMTS = [O.E4M3, O.E5M2, O.E2M1, O.E2M3, O.E3M2, O.INT8]
MODES = [O.FLOOR, O.ROUNDUP]


def rand_blocks(n=4000, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 32)) * np.exp2(rng.integers(-30, 30, size=(n, 1)))
    x[::7, 5] = 0.0
    x[::11, 9] = -0.0
    return x.astype(np.float32).astype(np.float64)


def q(x, fmt, mode):
    return O.quantize_blocks(x, fmt, mode)


def dq(codes, scales, fmt):
    codes = O.pack_codes(codes, fmt)
    return O.dequantize(codes, scales.reshape(-1, 1), fmt, "f32").view(np.float32).astype(np.float64)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
@pytest.mark.parametrize("mode", MODES, ids=["floor", "roundup"])
def test_value_idempotence(fmt, mode):
    x = rand_blocks()
    y = dq(*q(x, fmt, mode), fmt)
    z = dq(*q(y, fmt, mode), fmt)
    assert np.array_equal(y, z)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_code_idempotence_floor(fmt):
    x = rand_blocks()
    c1, s1 = q(x, fmt, O.FLOOR)
    c2, s2 = q(dq(c1, s1, fmt), fmt, O.FLOOR)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
@pytest.mark.parametrize("mode", MODES, ids=["floor", "roundup"])
def test_sign_symmetry(fmt, mode):
    x = rand_blocks()
    c1, s1 = q(x, fmt, mode)
    c2, s2 = q(-x, fmt, mode)
    assert np.array_equal(s1, s2)
    if fmt.integer:                                   # two's complement: code(-x) = -code(x)
        assert np.array_equal((-c1.astype(np.int64)) & 0xFF, c2)
    else:
        assert np.array_equal(c1 ^ (1 << (fmt.bits - 1)), c2)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
@pytest.mark.parametrize("mode", MODES, ids=["floor", "roundup"])
def test_power_of_two_equivariance(fmt, mode):
    x = rand_blocks()
    c1, s1 = q(x, fmt, mode)
    for j in (-5, 1, 7):
        c2, s2 = q(np.ldexp(x, j), fmt, mode)
        free = (s1.astype(int) + j >= 1) & (s1.astype(int) + j <= 254) & (s1 >= 1)
        assert np.array_equal(c1[free], c2[free])
        assert np.array_equal(s1[free].astype(int) + j, s2[free].astype(int))


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
@pytest.mark.parametrize("mode", MODES, ids=["floor", "roundup"])
def test_error_bound(fmt, mode):
    # RNE to m mantissa bits: relative error <= 2^-(m+1) while the scaled value
    # is in the format's normal range and not clipped.
    x = rand_blocks()
    c, s = q(x, fmt, mode)
    y = dq(c, s, fmt)
    e = s.astype(np.int64).reshape(-1, 1) - 127
    sv = np.abs(np.ldexp(x, -e))
    # INT8 (k / 64) behaves as 6 fraction bits on [1, 2), its top binade
    m, vmin_normal = (fmt.bias, 1.0) if fmt.integer else (fmt.mbits, 2.0 ** (1 - fmt.bias))
    ok = (sv >= vmin_normal) & (sv <= O.max_finite(fmt))
    assert ok.sum() > 1000
    rel = np.abs(y - x)[ok] / np.abs(x)[ok]
    assert rel.max() <= 2.0 ** -(m + 1)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_column_copy_orientation_closed_form(fmt):
    """X[r][c] = 2^(c % 8 - 3) * ((r % 32) + 1) / 32. Column c's blocks have max
    2^(c%8-3), so their floor scale code is c%8 - 3 - emax + 127; row r's blocks
    have max 2^4 * (r%32+1) / 32, so their code is floor(log2 of that) - emax + 127.
    A transposed or mis-indexed column plane fails this."""
    R, C = 64, 96
    r = np.arange(R).reshape(-1, 1)
    c = np.arange(C).reshape(1, -1)
    x = np.ldexp(((r % 32) + 1) / 32.0, (c % 8) - 3).astype(np.float32)
    em = O.emax_of(fmt)
    out = O.quantize(x, "f32", fmt, O.FLOOR, O.BOTH)
    exp_col = ((np.arange(C) % 8) - 3 - em + 127).reshape(C, 1).repeat(R // 32, axis=1)
    assert np.array_equal(out["col_scales"][0], exp_col)
    rowmax = 2.0 ** 4 * ((np.arange(R) % 32) + 1) / 32.0
    exp_row = (np.floor(np.log2(rowmax)).astype(int) - em + 127).reshape(R, 1).repeat(C // 32, axis=1)
    assert np.array_equal(out["row_scales"][0], exp_row)
    # column copy == row-wise quantization of the transpose
    t = O.quantize(np.ascontiguousarray(x.T), "f32", fmt, O.FLOOR, O.ROW)
    assert np.array_equal(t["row_codes"], out["col_codes"])
    assert np.array_equal(t["row_scales"], out["col_scales"])


def test_e2m1_nibble_order():
    # element 2k -> bits 3:0, element 2k+1 -> bits 7:4
    x = np.zeros(32, dtype=np.float32)
    x[0], x[1], x[2], x[3] = 0.5, 1.0, -6.0, 3.0
    x[31] = 4.0                                       # amax 6 -> scale 2^0 under both rules
    out = O.quantize(x.reshape(1, 32), "f32", O.E2M1, O.FLOOR, O.ROW)
    assert out["row_scales"][0, 0, 0] == 127
    b = out["row_codes"][0, 0]
    assert b.shape == (16,)
    assert b[0] == 0x21 and b[1] == 0x5F and b[15] == 0x60
    assert np.array_equal(O.unpack_e2m1(b)[:4], [1, 2, 0xF, 5])


def test_batched_layout_is_per_slice():
    x = I.to_bits(I.wide_range(0, 64, 96)).reshape(2, 32, 96)
    out = O.quantize(x, "bf16", O.E4M3, O.FLOOR, O.BOTH)
    for b in range(2):
        one = O.quantize(x[b], "bf16", O.E4M3, O.FLOOR, O.BOTH)
        for k in out:
            assert np.array_equal(out[k][b], one[k][0])
