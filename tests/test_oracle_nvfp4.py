"""Pins of the oracle's NVFP4 cast ("MXFP4 と NVFP4 は何が違うのか調べてみた" §3, §4
table and §7).

Independent references: the page's formulas and sizes (16-element blocks, 72
bits per block, the global scale = tensor amax / (6 * 448), an unsigned block
scale), torch's float32 arithmetic and float8_e4m3fn cast for the scale steps,
exact closed forms for tensors built around a known amax, and error bounds.
"""
import numpy as np
import pytest
import torch

import oracle as O


def rand(shape, seed, lo=-8, hi=8):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape) * np.exp2(rng.integers(lo, hi, size=shape[:-1] + (1,)))
    return x.astype(np.float32)


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
    # §3: the FP32 global scale is the tensor's largest magnitude over 6 * 448
    for a in (2688.0, 2688.0 * 2 ** -10, 1.0, 3.3e38, 1e-30, 123.456):
        x = np.zeros((1, 16, 32), np.float32)
        x[0, 3, 7] = -a
        x[0, 5, 9] = a / 3
        g = O.nvfp4_quantize(x, "f32", O.ROW)["global_scale"][0]
        ref = (torch.tensor(np.float32(a)) / 2688.0).item()     # torch's FP32 division
        assert g == np.float32(ref), a
    assert O.nvfp4_quantize(np.full((1, 16, 16), 2688.0, np.float32), "f32", O.ROW)["global_scale"][0] == 1.0


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


def test_scale_steps_match_torch_float32():
    """Block scale codes from torch: (amax/6)/g in float32, clamped to 448, cast
    to float8_e4m3fn (RNE)."""
    x = rand((1, 128, 256), 3, -12, 12)
    q = O.nvfp4_quantize(x, "f32", O.ROW)
    xt = torch.from_numpy(x[0])
    g = torch.tensor(q["global_scale"][0])
    amax = xt.abs().view(128, 16, 16).amax(dim=2)
    t = (amax / 6.0) / g
    ref = t.clamp(max=448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q["row_scales"][0], ref)
    # elements: fp32(x * fp32(1 / fp32(s * g))), RNE onto E2M1 (the pinned MX encoder)
    s = ref.astype(np.int64)
    sv = torch.from_numpy(O.value_table(O.E4M3)[s].astype(np.float32))
    rb = (1.0 / (sv * g)).repeat_interleave(16, dim=1)
    qv = (xt * rb).numpy().astype(np.float64)
    codes = O.encode_elements(qv, O.E2M1)
    codes[np.repeat(s == 0, 16, axis=1)] = 0
    assert np.array_equal(O.unpack_e2m1(q["row_codes"])[0], codes)


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


def test_zero_tensor_and_special_blocks():
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


def test_dequant_is_two_fp32_products():
    rng = np.random.default_rng(8)
    codes = rng.integers(0, 256, (1, 4, 16), dtype=np.uint8)      # 4 x 32 elements
    scales = rng.integers(0, 0x7F, (1, 4, 2), dtype=np.uint8)
    g = np.array([np.float32(1.7e-3)], np.float32)
    y = O.nvfp4_dequantize(codes, scales, g, "f32").view(np.float32)[0]
    c = O.unpack_e2m1(codes)[0]
    for r in range(4):
        for k in range(32):
            e = np.float32(O.decode_code(O.E2M1, int(c[r, k])))
            sv = np.float32(O.decode_code(O.E4M3, int(scales[0, r, k // 16])))
            ref = (torch.tensor(e) * torch.tensor(sv)) * torch.tensor(g[0])
            assert y[r, k] == ref.item() or (y[r, k] == 0 and ref.item() == 0)
