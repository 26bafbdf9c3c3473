"""Pins of the oracle's dequantization and output rounding."""
import math

import numpy as np
import pytest
import torch

import oracle as O

FMTS = [O.E4M3, O.E5M2, O.E2M1, O.E2M3, O.E3M2, O.INT8]


def all_code_scale_pairs(fmt):
    ncode = 1 << fmt.bits
    codes = np.tile(np.arange(ncode, dtype=np.uint8), 256)
    scales = np.repeat(np.arange(256, dtype=np.uint8), ncode)
    pad = (-codes.size) % 32
    codes = np.concatenate([codes, np.zeros(pad, np.uint8)])
    scales = np.concatenate([scales, np.full(pad, 127, np.uint8)])
    # one scale per element: lay each pair out as its own 32-block (code in slot 0)
    blocks = np.zeros((codes.size, 32), dtype=np.uint8)
    blocks[:, 0] = codes
    return blocks, scales.reshape(-1, 1)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_f32_output_is_exact_exponent_add(fmt):
    # "MXFP4 と NVFP4 は何が違うのか調べてみた" §7: applying an E8M0 scale is an
    # exponent add with no rounding error.
    blocks, scales = all_code_scale_pairs(fmt)
    packed = O.pack_codes(blocks, fmt)
    y = O.dequantize(packed, scales, fmt, "f32")[:, 0]
    for code, k, bits in zip(blocks[:, 0], scales[:, 0], y):
        v = O.decode_code(fmt, int(code))
        if k == 255 or math.isnan(v):
            assert bits == 0x7FC00000
            continue
        with np.errstate(over="ignore"):
            ref = np.float32(math.ldexp(v, int(k) - 127))    # the exact product fits FP32...
        if math.isfinite(math.ldexp(v, int(k) - 127)) and abs(math.ldexp(v, int(k) - 127)) < 2.0 ** 128:
            assert float(ref) == math.ldexp(v, int(k) - 127)  # ...bit for bit
        assert bits == ref.view(np.uint32), (code, k)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_bf16_output_matches_torch_rounding(fmt):
    blocks, scales = all_code_scale_pairs(fmt)
    packed = O.pack_codes(blocks, fmt)
    f = O.dequantize(packed, scales, fmt, "f32")[:, 0].view(np.float32)
    b = O.dequantize(packed, scales, fmt, "bf16")[:, 0]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(f)
    assert (b[nan] == 0x7FC0).all()
    assert np.array_equal(b[~nan], ref[~nan])


def test_round_to_binary_matches_numpy_float32_cast():
    rng = np.random.default_rng(3)
    v = rng.standard_normal(200000) * np.exp2(rng.integers(-160, 135, size=200000))
    v = np.concatenate([v, [3.4028235677973366e38, 3.4028235677973366e38 * (1 + 2 ** -25), 2.0 ** -150,
                            2.0 ** -149 * 1.5, 2.0 ** -149 * 2.5, -0.0, 0.0]])
    with np.errstate(over="ignore"):
        ref = v.astype(np.float32).astype(np.float64)
    ours = O.round_to_binary(v, 23, -126, 127)
    assert np.array_equal(np.signbit(ours), np.signbit(ref))
    assert np.array_equal(ours, ref)


def test_round_to_binary_matches_torch_bf16_cast():
    rng = np.random.default_rng(4)
    bits = rng.integers(0, 1 << 32, size=300000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    ours = O.round_to_binary(f.astype(np.float64), 7, -126, 127)
    assert np.array_equal(ours, ref)


def test_overflow_at_top_of_range_is_inf():
    # round-up rule with a block max within one E4M3 step of 2^128: the scaled
    # max rounds up to 256 (tie to even) and the dequantized value is 2^128,
    # which overflows FP32 to +Inf under round-to-nearest.
    blk = np.zeros((1, 32))
    blk[0, 0] = 1.9375 * 2.0 ** 127
    codes, scales = O.quantize_blocks(blk, O.E4M3, O.ROUNDUP)
    assert scales[0] == 127 + 120
    assert O.decode_code(O.E4M3, int(codes[0, 0])) == 256.0
    y = O.dequantize(codes, scales.reshape(1, 1), O.E4M3, "f32").view(np.float32)
    assert y[0, 0] == np.inf


def test_e5m2_inf_codes_and_nan_codes():
    codes = np.zeros((1, 32), dtype=np.uint8)
    codes[0, :6] = [0x7C, 0xFC, 0x7D, 0xFF, 0x7B, 0xFB]
    y = O.dequantize(codes, np.array([[127]], np.uint8), O.E5M2, "f32")[0]
    assert y[0] == 0x7F800000 and y[1] == 0xFF800000
    assert y[2] == 0x7FC00000 and y[3] == 0x7FC00000
    assert y[4] == np.float32(57344.0).view(np.uint32) and y[5] == np.float32(-57344.0).view(np.uint32)
