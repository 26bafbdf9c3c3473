"""Pins for the FP4-in-FP8 nested requantization oracle ([Q] §6, DeepSeek-V4's
nested structure): the 512-tiles-per-block count, exactness below the spread
threshold by exhaustive membership in the E4M3 value set, the exact failures
just above it, scale equivariance, the active-sub-block rule, and the full
pipeline from FP32 weights through MXFP4."""
import numpy as np
import pytest

import oracle as O

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

E4M3_VALUES = set(float(v) for v in O.value_table(O.E4M3) if np.isfinite(v))
E2M1_VALUES = O.value_table(O.E2M1)


def mxfp4_plane(rng, r, c, kbase, spread_max, zero_frac=0.0):
    """Random MXFP4 plane: codes [r][c/2], scales [r][c/32] drawn per 128x128
    block from [kb, kb + spread_max] with kb = kbase per block."""
    q = rng.integers(0, 16, (r, c)).astype(np.uint8)
    if zero_frac:
        z = rng.random((r, c // 32)) < zero_frac
        q.reshape(r, c // 32, 32)[z] = rng.choice([0, 8], size=(z.sum(), 32)).astype(np.uint8)
    k = kbase + rng.integers(0, spread_max + 1, (r, c // 32))
    return O.pack_e2m1(q), k.astype(np.uint8)


def mx_values(codes, scales):
    """float64 values of an MXFP4 plane (E2M1 value x 2^(k-127)), from the tables."""
    q = O.unpack_e2m1(codes)
    k = np.repeat(np.asarray(scales, np.int64), 32, axis=-1)
    return E2M1_VALUES[q] * np.ldexp(1.0, k - 127)


def test_512_subtiles_per_block():
    """[Q] §6: a 128x128 FP8 tile holds 4 x 128 = 512 tiles of 1x32."""
    assert O.SUBS_PER_FP8_BLOCK == 4 * 128 == 512
    codes = np.full((128, 64), 0x11, np.uint8)                    # every element 0.5
    scales = np.full((128, 4), 100, np.uint8)
    scales.reshape(-1)[7] = 90                                    # exactly one sub-block is the minimum
    out = O.requant_fp4_to_fp8(codes, scales)
    assert out["spread"].shape == (1, 1) and out["spread"][0, 0] == 10
    # all 512 sub-blocks count: raising any single one of them changes kmax
    for i in range(0, 512, 37):
        s2 = scales.copy()
        s2.reshape(-1)[i] = 105
        assert O.requant_fp4_to_fp8(codes, s2)["spread"][0, 0] == (105 - 90 if i != 7 else 0)


def test_e4m3_has_two_more_exponent_bits():
    """[Q] §6: the width difference the losslessness argument rests on."""
    assert O.E4M3.ebits - O.E2M1.ebits == 2


def test_threshold_is_exact_by_membership():
    """Every E2M1 value times 2^E is an E4M3 value for E in [-8, 6] (checked by
    membership in the decoded E4M3 set); E = -9 loses 0.5 and 1.5, E = 7 loses 4 and 6."""
    ok = [all(float(v) * 2.0 ** e in E4M3_VALUES for v in E2M1_VALUES) for e in range(-12, 10)]
    assert [e for e, g in zip(range(-12, 10), ok) if g] == list(range(-8, 7))
    lost_low = sorted({abs(float(v)) for v in E2M1_VALUES if float(v) * 2.0 ** -9 not in E4M3_VALUES})
    assert lost_low == [0.5, 1.5]
    lost_high = sorted({abs(float(v)) for v in E2M1_VALUES if float(v) * 2.0 ** 7 not in E4M3_VALUES})
    assert lost_high == [4.0, 6.0]                                # 512 and 768 exceed 448
    assert O.LOSSLESS_SPREAD == 6 - (-8)


@pytest.mark.parametrize("spread_max", [0, 5, 14])
def test_lossless_below_threshold(spread_max):
    """The pages' claim: with the scale ratio under the threshold, the FP8 copy
    decodes to exactly the MXFP4 values."""
    rng = np.random.default_rng(spread_max)
    for kbase in (0, 60, 127, 240 - spread_max):
        codes, scales = mxfp4_plane(rng, 256, 384, kbase, spread_max)
        out = O.requant_fp4_to_fp8(codes, scales)
        assert out["spread"].max() <= spread_max
        got = O.dequantize_fp8_blocks(out["e4m3"], out["block_scale"])
        exp = mx_values(codes, scales)
        assert np.array_equal(got, exp)
        assert np.array_equal(np.signbit(got), np.signbit(exp))     # signed zeros survive


def test_spread_15_loses_exactly_the_predicted_elements():
    rng = np.random.default_rng(15)
    codes, scales = mxfp4_plane(rng, 128, 128, 100, 0)
    scales[:] = 115
    scales[3, 1] = 100                                            # one sub-block 15 binades down
    out = O.requant_fp4_to_fp8(codes, scales)
    assert out["spread"][0, 0] == 15
    got = O.dequantize_fp8_blocks(out["e4m3"], out["block_scale"])
    exp = mx_values(codes, scales)
    bad = got != exp
    q = O.unpack_e2m1(codes)
    predicted = np.zeros_like(bad)
    predicted[3, 32:64] = np.isin(q[3, 32:64] & 7, [1, 3])        # 0.5 and 1.5
    assert np.array_equal(bad, predicted) and bad.any()
    # nearest-even onto E4M3's 2^-9 grid: 0.5 * 2^-9 -> 0, 1.5 * 2^-9 -> 2^-8
    s = float(out["block_scale"][0, 0])
    for code, want in ((1, 0.0), (3, 2.0 ** -8), (9, -0.0), (11, -(2.0 ** -8))):
        cols = np.where(q[3, 32:64] == code)[0]
        if cols.size:
            v = got[3, 32 + cols[0]] / s
            assert v == want and np.signbit(v) == np.signbit(want)


def test_block_scale_places_the_largest_value_at_384():
    codes = np.full((128, 64), 0x77, np.uint8)                    # every element 6
    for k in (0, 5, 6, 127, 200, 254):
        out = O.requant_fp4_to_fp8(codes, np.full((128, 4), k, np.uint8))
        assert out["block_scale"][0, 0] == np.float32(2.0 ** (k - 133))
        assert (O.value_table(O.E4M3)[out["e4m3"]] == 384.0).all()


def test_scale_equivariance():
    """Adding j to every scale code leaves the E4M3 codes and spreads alone and
    multiplies the block scales by 2^j."""
    rng = np.random.default_rng(5)
    codes, scales = mxfp4_plane(rng, 200, 288, 50, 20, zero_frac=0.1)
    a = O.requant_fp4_to_fp8(codes, scales)
    for j in (-50, 3, 100):
        b = O.requant_fp4_to_fp8(codes, (scales.astype(int) + j).astype(np.uint8))
        assert np.array_equal(a["e4m3"], b["e4m3"]) and np.array_equal(a["spread"], b["spread"])
        assert np.array_equal(b["block_scale"], (a["block_scale"].astype(np.float64) * 2.0 ** j).astype(np.float32))


def test_zero_and_nan_subblocks_do_not_count():
    codes = np.full((128, 64), 0x22, np.uint8)                    # every element 1.0
    scales = np.full((128, 4), 120, np.uint8)
    codes[5, 0:16] = 0x80                                         # sub-block (5, 0): only -0 and +0
    scales[5, 0] = 0                                              # the scale a zero block gets
    scales[9, 2] = 0xFF                                           # NaN sub-block
    scales[17, 3] = 250                                           # all-zero sub-block with a big scale
    codes[17, 48:64] = 0x00
    out = O.requant_fp4_to_fp8(codes, scales)
    assert out["spread"][0, 0] == 0 and out["block_scale"][0, 0] == np.float32(2.0 ** (120 - 133))
    e = out["e4m3"]
    assert (e[9, 64:96] == 0x7F).all()
    assert (e[5, 0:32] == np.tile([0x00, 0x80], 16)).all()
    assert (e[17, 96:128] == 0).all()
    empty = O.requant_fp4_to_fp8(np.zeros((128, 64), np.uint8), np.zeros((128, 4), np.uint8))
    assert empty["spread"][0, 0] == 0 and empty["block_scale"][0, 0] == 1.0 and (empty["e4m3"] == 0).all()


def test_ragged_blocks_and_transpose():
    rng = np.random.default_rng(7)
    codes, scales = mxfp4_plane(rng, 200, 160, 90, 9)             # blocks 2 x 2, the last ones partial
    out = O.requant_fp4_to_fp8(codes, scales)
    assert out["e4m3"].shape == (200, 160) and out["block_scale"].shape == (2, 2)
    k = scales.astype(int)
    for br, bc, rows, subs in ((0, 0, slice(0, 128), slice(0, 4)), (1, 1, slice(128, 200), slice(4, 5))):
        kk = k[rows, subs]
        assert out["spread"][br, bc] == kk.max() - kk.min()
    assert np.array_equal(out["e4m3_t"], out["e4m3"].T)
    assert np.array_equal(out["block_scale_t"], out["block_scale"].T)
    assert np.array_equal(O.dequantize_fp8_blocks(out["e4m3"], out["block_scale"]), mx_values(codes, scales))


def test_batch_slices_are_independent():
    rng = np.random.default_rng(8)
    parts = [mxfp4_plane(rng, 128, 256, 40 + 30 * i, 12) for i in range(3)]
    codes = np.stack([p[0] for p in parts])
    scales = np.stack([p[1] for p in parts])
    out = O.requant_fp4_to_fp8(codes, scales)
    for i, (c, s) in enumerate(parts):
        one = O.requant_fp4_to_fp8(c, s)
        for key in ("e4m3", "block_scale", "spread"):
            assert np.array_equal(out[key][i], one[key])


def test_pipeline_from_fp32_weights():
    """FP32 master -> MXFP4 (floor rule) -> FP8: weights whose blocks span few
    binades come back exactly; a block holding a tiny-scaled tile reports a
    spread beyond the threshold and loses only where predicted."""
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((256, 256)) * 0.02).astype(np.float32)
    q = O.quantize(w, "f32", O.E2M1, O.FLOOR, O.ROW)
    out = O.requant_fp4_to_fp8(q["row_codes"][0], q["row_scales"][0])
    assert out["spread"].max() <= O.LOSSLESS_SPREAD
    assert np.array_equal(O.dequantize_fp8_blocks(out["e4m3"], out["block_scale"]),
                          mx_values(q["row_codes"][0], q["row_scales"][0]))
    w[0, :32] *= 2.0 ** -20
    q = O.quantize(w, "f32", O.E2M1, O.FLOOR, O.ROW)
    out = O.requant_fp4_to_fp8(q["row_codes"][0], q["row_scales"][0])
    assert out["spread"][0, 0] > O.LOSSLESS_SPREAD
    bad = O.dequantize_fp8_blocks(out["e4m3"], out["block_scale"]) != mx_values(q["row_codes"][0], q["row_scales"][0])
    assert bad[1:].sum() == 0 and bad[0, 32:].sum() == 0 and bad[0, :32].any()
