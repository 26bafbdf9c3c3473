"""Bit-exact parity of the FP4-in-FP8 requantization (mx_requant_fp4_fp8) with
the CPU oracle: E4M3 codes, block scales (FP32 bits), spreads and the
transposed copy."""
import numpy as np
import pytest
import torch

import mx_inputs as I
import oracle as O

pytestmark = pytest.mark.gpu


def plane(rng, b, r, c, kbase, spread, zero_frac=0.05, nan_frac=0.0):
    """Random MXFP4 plane [b][r][c/2] + [b][r][c/32]: scale codes in
    [kbase, kbase + spread], some all-zero sub-blocks (with arbitrary scales),
    some NaN sub-blocks."""
    q = rng.integers(0, 16, (b, r, c)).astype(np.uint8)
    k = (kbase + rng.integers(0, spread + 1, (b, r, c // 32))).clip(0, 254).astype(np.uint8)
    z = rng.random((b, r, c // 32)) < zero_frac
    q.reshape(b, r, c // 32, 32)[z] = rng.choice([0, 8], size=(int(z.sum()), 32)).astype(np.uint8)
    zk = z & (rng.random(z.shape) < 0.5)                          # zero sub-blocks with any scale
    k[zk] = rng.integers(0, 255, int(zk.sum()), dtype=np.uint8)
    k[rng.random(k.shape) < nan_frac] = 0xFF
    return O.pack_e2m1(q), k


def run(mx, codes, scales, shape, axis):
    out = mx.mx_requant_fp4_fp8(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), shape, axis)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def compare(got, exp, axis, what):
    keys = ["spread"]
    if axis in ("row", "both"):
        keys += ["e4m3", "block_scale"]
    if axis in ("col", "both"):
        keys += ["e4m3_t", "block_scale_t"]
    for key in keys:
        g, e = got[key], exp[key]
        if key.startswith("block_scale"):
            g, e = g.view(np.uint32), e.view(np.uint32)
        assert g.shape == e.shape, (what, key, g.shape, e.shape)
        bad = np.argwhere(g != e)
        if bad.size:
            idx = tuple(bad[0])
            raise AssertionError(f"{what} {key}: {len(bad)} mismatches, first at {idx}: gpu={g[idx]:#x} "
                                 f"oracle={e[idx]:#x}")


def check(mx, codes, scales, axis, what=""):
    b, r, c2 = codes.shape
    got = run(mx, codes, scales, (b, r, 2 * c2), axis)
    exp = O.requant_fp4_to_fp8(codes, scales)
    compare(got, exp, axis, what)
    return got, exp


@pytest.mark.parametrize("axis", ["row", "col", "both"])
def test_shapes_and_ragged_edges(mx, axis):
    rng = np.random.default_rng(71)
    for b, r, c in [(1, 128, 256), (1, 208, 160), (3, 256, 384), (1, 64, 96), (1, 16, 32), (2, 272, 4128),
                    (1, 400, 544)]:
        codes, scales = plane(rng, b, r, c, 100, 12, nan_frac=0.002)
        check(mx, codes, scales, axis, f"{(b, r, c)}")


def test_scale_words_batches_and_ragged_rows(mx):
    """Both copies with cols % 256 == 0 load each tile's scales as one dword per
    thread through LDS: batches, ragged last tile rows (272 and 64 rows) and
    several tile columns, with NaN-scale sub-blocks."""
    rng = np.random.default_rng(74)
    for b, r, c in [(2, 272, 512), (3, 64, 768), (1, 400, 1024)]:
        codes, scales = plane(rng, b, r, c, 100, 12, nan_frac=0.002)
        check(mx, codes, scales, "both", f"{(b, r, c)}")


@pytest.mark.parametrize("axis", ["row", "col", "both"])
def test_xcd_tile_row_order(mx, axis):
    """When batch * ceil(rows / 128) is a multiple of 8, each XCD takes whole tile
    rows (tile row t on XCD t mod 8): batches, ragged last tile rows and columns,
    narrow tensors, outputs that start as a sentinel (a tile left unwritten or
    written twice to the wrong place shows up)."""
    rng = np.random.default_rng(75)
    for b, r, c in [(2, 512, 4128), (8, 112, 256), (1, 1024, 96), (4, 272, 544), (2, 4096, 512)]:
        codes, scales = plane(rng, b, r, c, 100, 12, nan_frac=0.002)
        nbr, nbc = -(-r // 128), -(-c // 128)
        out = {}
        if axis in ("row", "both"):
            out["e4m3"] = torch.full((b, r, c), 0xA5, dtype=torch.uint8, device="cuda")
            out["block_scale"] = torch.full((b, nbr, nbc), -1.0, dtype=torch.float32, device="cuda")
        if axis in ("col", "both"):
            out["e4m3_t"] = torch.full((b, c, r), 0xA5, dtype=torch.uint8, device="cuda")
            out["block_scale_t"] = torch.full((b, nbc, nbr), -1.0, dtype=torch.float32, device="cuda")
        out["spread"] = torch.full((b, nbr, nbc), 0xA5, dtype=torch.uint8, device="cuda")
        got = mx.mx_requant_fp4_fp8(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), (b, r, c), axis,
                                    out=out)
        torch.cuda.synchronize()
        compare({k: v.cpu().numpy() for k, v in got.items()}, O.requant_fp4_to_fp8(codes, scales), axis,
                f"{(b, r, c)}")


def test_row_copy_accepts_any_row_count(mx):
    rng = np.random.default_rng(72)
    for r in (1, 37, 129, 255):
        codes, scales = plane(rng, 1, r, 320, 60, 9)
        check(mx, codes, scales, "row", f"rows={r}")


@pytest.mark.parametrize("spread", [0, 14, 15, 20, 60])
def test_spreads_across_the_threshold(mx, spread):
    rng = np.random.default_rng(73 + spread)
    codes, scales = plane(rng, 2, 256, 512, 120 - spread // 2, spread)
    got, exp = check(mx, codes, scales, "both", f"spread {spread}")
    assert got["spread"].max() <= spread
    # blocks whose spread is within the threshold converted exactly
    e2m1 = O.value_table(O.E2M1)[O.unpack_e2m1(codes)]
    kk = np.repeat(scales.astype(np.int64), 32, axis=-1)
    mxv = np.where(kk == 0xFF, np.nan, e2m1 * np.ldexp(1.0, np.where(kk == 0xFF, 0, kk) - 127))
    fp8v = O.dequantize_fp8_blocks(got["e4m3"], got["block_scale"])
    ok = np.repeat(np.repeat(got["spread"] <= O.LOSSLESS_SPREAD, 128, axis=-2), 128, axis=-1)
    fin = ~np.isnan(mxv)
    assert np.array_equal(fp8v[ok & fin], mxv[ok & fin])


def test_every_code_at_every_shift(mx):
    """Every E2M1 code in sub-blocks 0 .. 40 binades below the block's largest,
    for block maxima from the bottom to the top of the E8M0 range (subnormal
    FP32 block scales included), with NaN and all-zero sub-blocks."""
    rows = []
    for kmax in (0, 3, 6, 7, 40, 127, 200, 254):
        blk = np.zeros((128, 128), np.uint8)
        blk[:] = np.tile(np.arange(16, dtype=np.uint8), 8)
        k = np.empty((128, 4), np.int64)
        k[:] = kmax - (np.arange(128 * 4).reshape(128, 4) % 41)
        k = k.clip(0, 254)
        k[0, 0] = kmax
        k[5, 1] = 0xFF
        blk[9, 64:96] = 8                                         # an all -0 sub-block ...
        k[9, 2] = min(kmax + 30, 254)                             # ... with a scale above kmax
        rows.append((O.pack_e2m1(blk), k.astype(np.uint8)))
    codes = np.concatenate([r[0] for r in rows])[None]
    scales = np.concatenate([r[1] for r in rows])[None]
    check(mx, codes, scales, "both", "every code")


def test_all_zero_and_all_nan_blocks(mx):
    codes = np.zeros((1, 256, 128), np.uint8)
    scales = np.zeros((1, 256, 8), np.uint8)
    scales[0, 128:, :] = 0xFF
    codes[0, 200, 10] = 0x30                                      # one nonzero code in a NaN sub-block
    got, _ = check(mx, codes, scales, "both", "empty")
    assert (got["block_scale"] == 1.0).all() and (got["spread"] == 0).all()


def test_pipeline_from_gpu_mxfp4(mx):
    """FP32 weights -> mx_quantize (E2M1, floor, rows) -> mx_requant_fp4_fp8,
    everything on the GPU; the oracle requantizes the same MXFP4 planes."""
    w = I.weights(384, 640, seed=74).float().cuda()
    q = mx.mx_quantize(w, "e2m1", "floor", "row")
    torch.cuda.synchronize()
    codes, scales = q["row_codes"].cpu().numpy()[None], q["row_scales"].cpu().numpy()[None]
    got, exp = check(mx, codes, scales, "both", "pipeline")
    assert (got["spread"] <= O.LOSSLESS_SPREAD).all()


# (the 14336x4096 requantization is compared whole in test_gpu_full.py)


# ---------------- one pass from the master weights ----------------

OMODE = {"floor": O.FLOOR, "roundup": O.ROUNDUP}


def qat_oracle(x, mode):
    dt = "bf16" if x.dtype == torch.bfloat16 else "f32"
    q = O.quantize(I.to_bits(x), dt, O.E2M1, OMODE[mode], O.ROW)
    exp = O.requant_fp4_to_fp8(q["row_codes"], q["row_scales"])
    exp["fp4_codes"], exp["fp4_scales"] = q["row_codes"], q["row_scales"]
    if x.dim() == 2:
        exp = {k: v[0] for k, v in exp.items()}
    return exp


def check_qat(mx, x, mode, axis, what):
    out = mx.mx_quantize_fp4_fp8(x.cuda().contiguous(), mode, axis)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in out.items()}
    exp = qat_oracle(x, mode)
    compare(got, exp, axis, what)
    for key in ("fp4_codes", "fp4_scales"):
        assert np.array_equal(got[key], exp[key]), (what, key)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["floor", "roundup"])
@pytest.mark.parametrize("axis", ["row", "col", "both"])
def test_qat_shapes(mx, axis, mode, dt):
    for b, r, c in [(1, 128, 256), (1, 208, 160), (2, 272, 544), (1, 16, 32), (1, 400, 4128)]:
        x = torch.stack([I.weights(r, c, seed=80 + i) for i in range(b)])
        x = x.float() if dt == "f32" else x
        check_qat(mx, x if b > 1 else x[0], mode, axis, f"{(b, r, c)}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_qat_specials_and_wide_range(mx, dt):
    g = I.gradients(288, 320, seed=81)                           # zeros, NaN, Inf, zero blocks
    check_qat(mx, g if dt == "f32" else g.to(torch.bfloat16), "floor", "both", "gradients")
    w = torch.stack([I.wide_range(i, 256, 384, seed=82) for i in range(2)])
    check_qat(mx, w.float() if dt == "f32" else w, "roundup", "both", "wide range")
    e = I.fp32_edges("e2m1")
    e = e[: (e.shape[0] // 16) * 16]
    check_qat(mx, e if dt == "f32" else e.to(torch.bfloat16), "floor", "both", "edges")


def test_qat_equals_the_two_calls(mx):
    x = I.weights(512, 768, seed=83).float().cuda()
    one = mx.mx_quantize_fp4_fp8(x, "floor", "both")
    q = mx.mx_quantize(x, "e2m1", "floor", "row")
    two = mx.mx_requant_fp4_fp8(q["row_codes"], q["row_scales"], (512, 768), "both")
    torch.cuda.synchronize()
    assert torch.equal(one["fp4_codes"], q["row_codes"]) and torch.equal(one["fp4_scales"], q["row_scales"])
    for k in ("e4m3", "block_scale", "e4m3_t", "block_scale_t", "spread"):
        assert torch.equal(one[k], two[k]), k


# (the 14336x4096 FP32 master-weight pass is compared whole in test_gpu_full.py)
