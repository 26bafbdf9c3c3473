"""Bit-exact parity of the HIP path (through the C ABI) with the CPU oracle.

Codes and scales must match exactly; dequantized outputs must match bit for
bit (NaN is canonical on both sides). Inputs come from mx_inputs only.
"""
import numpy as np
import pytest
import torch

import mx_inputs as I
import oracle as O

pytestmark = pytest.mark.gpu

OFMT = {"e4m3": O.E4M3, "e5m2": O.E5M2, "e2m1": O.E2M1, "e2m3": O.E2M3, "e3m2": O.E3M2, "int8": O.INT8}
OMODE = {"floor": O.FLOOR, "roundup": O.ROUNDUP}
OAXIS = {"row": O.ROW, "col": O.COL, "both": O.BOTH}
FMTS = ["e4m3", "e5m2", "e2m1", "e2m3", "e3m2", "int8"]
NEW_FMTS = ["e2m3", "e3m2", "int8"]          # the MXFP6 and MXINT8 rows of the family table
MODES = ["floor", "roundup"]


def gpu_quant(mx, x, fmt, mode, axis):
    out = mx.mx_quantize(x.cuda().contiguous(), fmt, mode, axis)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def oracle_quant(x, fmt, mode, axis):
    dt = "bf16" if x.dtype == torch.bfloat16 else "f32"
    out = O.quantize(I.to_bits(x), dt, OFMT[fmt], OMODE[mode], OAXIS[axis])
    if x.dim() == 2:
        out = {k: v[0] for k, v in out.items()}
    return out


def assert_same(got, exp, what=""):
    assert set(got) == set(exp), (got.keys(), exp.keys())
    for k in exp:
        g, e = got[k], exp[k]
        assert g.shape == e.shape, (what, k, g.shape, e.shape)
        bad = np.argwhere(g != e)
        if bad.size:
            idx = tuple(bad[0])
            raise AssertionError(f"{what} {k}: {len(bad)} mismatches, first at {idx}: "
                                 f"gpu={g[idx]:#x} oracle={e[idx]:#x}")


def check(mx, x, fmt, mode, axis, what=""):
    assert_same(gpu_quant(mx, x, fmt, mode, axis), oracle_quant(x, fmt, mode, axis), what)


def pad_rows(t, mult=32):
    pad = (-t.shape[0]) % mult
    if pad:
        t = torch.cat([t, torch.zeros((pad,) + tuple(t.shape[1:]), dtype=t.dtype)])
    return t


# ---------------- exhaustive and directed inputs ----------------

@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("fmt", FMTS)
def test_bf16_sweep_rows(mx, fmt, mode):
    """Every BF16 pattern under every reachable shared scale, blocks along rows."""
    check(mx, I.bf16_sweep(fmt), fmt, mode, "row", "sweep/row")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("fmt", FMTS)
def test_bf16_sweep_columns(mx, fmt, mode):
    """The same sweep with each block laid down a column (fused kernel, both planes)."""
    x = pad_rows(I.bf16_sweep(fmt)).T.contiguous()          # [32, n]
    check(mx, x, fmt, mode, "both", "sweep/col")


@pytest.mark.parametrize("axis", ["row", "col"])
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("fmt", FMTS)
def test_bf16_amax_sweep(mx, fmt, mode, axis):
    x = pad_rows(I.bf16_amax_sweep())
    if axis == "col":
        x = x.T.contiguous()
    check(mx, x, fmt, mode, axis, "amax")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("fmt", FMTS)
def test_edge_blocks(mx, fmt, mode, dt):
    x = I.fp32_edges(fmt) if dt == "f32" else I.bf16_edges(fmt)
    x = pad_rows(x)
    check(mx, x, fmt, mode, "row", "edges/row")
    check(mx, x.T.contiguous(), fmt, mode, "both", "edges/col")


# ---------------- workloads at small sizes (several tiles + ragged tails) ----------------

def test_fp32_normal_quant_dequant(mx):
    """256x1024 FP32 N(0,1), row-wise E4M3, floor rule, then dequantize to FP32."""
    x = I.fp32_normal(256, 1024, seed=0)
    got = gpu_quant(mx, x, "e4m3", "floor", "row")
    exp = oracle_quant(x, "e4m3", "floor", "row")
    assert_same(got, exp, "fp32_normal")
    rc = torch.from_numpy(got["row_codes"]).cuda()
    rs = torch.from_numpy(got["row_scales"]).cuda()
    y = mx.mx_dequantize(rc, rs, "e4m3", (256, 1024), "f32")
    torch.cuda.synchronize()
    ref = O.dequantize(exp["row_codes"], exp["row_scales"], O.E4M3, "f32")
    assert np.array_equal(y.cpu().numpy().view(np.uint32), ref)


@pytest.mark.parametrize("shape", [(544, 416), (128, 128), (32, 32), (96, 4128)])
def test_activations_fused(mx, shape):
    check(mx, I.activations(*shape, seed=11), "e4m3", "floor", "both", f"act{shape}")


@pytest.mark.parametrize("mode", MODES)
def test_weights_e2m1(mx, mode):
    x = I.weights(352, 288, seed=12)
    check(mx, x, "e2m1", mode, "row", "weights")
    check(mx, x, "e2m1", mode, "both", "weights/both")


@pytest.mark.parametrize("axis", ["col", "both"])
def test_gradients_e5m2(mx, axis):
    x = I.gradients(288, 352, seed=13)
    assert torch.isnan(x).any() or torch.isinf(x).any()
    check(mx, x, "e5m2", "roundup", axis, "grads")


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_wide_range_batch_round_trip(mx, out_dtype):
    b, r, c = 3, 160, 288
    x = torch.stack([I.wide_range(i, r, c, seed=14) for i in range(b)])
    got = gpu_quant(mx, x, "e4m3", "floor", "both")
    exp = oracle_quant(x, "e4m3", "floor", "both")
    assert_same(got, exp, "wide")
    for plane, shp in (("row", (b, r, c)), ("col", (b, c, r))):
        codes = torch.from_numpy(got[f"{plane}_codes"]).cuda()
        scales = torch.from_numpy(got[f"{plane}_scales"]).cuda()
        y = mx.mx_dequantize(codes, scales, "e4m3", shp, out_dtype)
        torch.cuda.synchronize()
        ref = O.dequantize(exp[f"{plane}_codes"], exp[f"{plane}_scales"], O.E4M3, out_dtype)
        yb = y.cpu().contiguous()
        yb = yb.view(torch.int16).numpy().view(np.uint16) if out_dtype == "bf16" else yb.numpy().view(np.uint32)
        assert np.array_equal(yb, ref), plane


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", FMTS)
def test_ragged_shapes(mx, fmt, dt):
    g = torch.Generator().manual_seed(21)
    shapes = [(1, 33, 32, "row"), (2, 64, 160, "both"), (1, 32, 32, "col"), (3, 96, 224, "both"),
              (1, 1, 4096, "row"), (2, 160, 96, "col"), (1, 257, 64, "row")]
    for b, r, c, axis in shapes:
        x = torch.randn((b, r, c), generator=g) * torch.exp2(torch.randint(-8, 8, (b, r, 1), generator=g).float())
        x = x.to(torch.bfloat16) if dt == "bf16" else x
        for mode in MODES:
            check(mx, x, fmt, mode, axis, f"ragged {(b, r, c, axis, mode)}")


@pytest.mark.parametrize("fmt", ["e4m3", "e2m3", "int8", "e2m1"])
def test_row_scale_words(mx, fmt):
    """Fused casts with cols % 256 == 0 store each tile row's 8 row-scale bytes
    as one word after the barrier: batches, a ragged last tile row (160 and
    4128 rows), sentinel-filled outputs, and a row-scale plane offset by 4 bytes
    (not 8-byte aligned), which must take the per-wave stores instead."""
    g = torch.Generator().manual_seed(31)
    bits = {"e4m3": 8, "e2m3": 6, "int8": 8, "e2m1": 4}[fmt]
    for b, r, c in [(2, 160, 512), (1, 4128, 256), (3, 64, 768)]:
        x = (torch.randn((b, r, c), generator=g) *
             torch.exp2(torch.randint(-10, 10, (b, r, c // 32), generator=g).float()).repeat_interleave(32, dim=2))
        x = x.to(torch.bfloat16)
        exp = oracle_quant(x, fmt, "floor", "both")
        for shift in (0, 4):
            rs = torch.full((b * r * (c // 32) + 8,), 0xA5, dtype=torch.uint8, device="cuda")
            out = {"row_codes": torch.full((b, r, c * bits // 8), 0xA5, dtype=torch.uint8, device="cuda"),
                   "row_scales": rs[shift:shift + b * r * (c // 32)].view(b, r, c // 32),
                   "col_codes": torch.full((b, c, r * bits // 8), 0xA5, dtype=torch.uint8, device="cuda"),
                   "col_scales": torch.full((b, c, r // 32), 0xA5, dtype=torch.uint8, device="cuda")}
            got = mx.mx_quantize(x.cuda(), fmt, "floor", "both", out=out)
            torch.cuda.synchronize()
            got = {k: v.cpu().numpy() for k, v in got.items()}
            assert_same(got, exp, f"row scale words {(b, r, c, fmt, shift)}")
            guard = rs.cpu().numpy()
            assert (guard[:shift] == 0xA5).all() and (guard[shift + b * r * (c // 32):] == 0xA5).all()


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
def test_fp6_row_lines(mx, fmt, dt):
    """Fused 6-bit casts with cols % 64 == 0 stage the row codes and write them
    as 16-byte chunks: tiles of 256, 64 and 192 columns (ragged last tiles), a
    batch, and outputs that start as a sentinel so that a chunk left unwritten
    shows up."""
    g = torch.Generator().manual_seed(29)
    for b, r, c in [(2, 96, 320), (1, 64, 64), (1, 128, 4160), (3, 32, 448)]:
        x = torch.randn((b, r, c), generator=g) * torch.exp2(torch.randint(-8, 8, (b, r, 1), generator=g).float())
        x = x.to(torch.bfloat16) if dt == "bf16" else x
        out = {"row_codes": torch.full((b, r, c * 3 // 4), 0xA5, dtype=torch.uint8, device="cuda"),
               "row_scales": torch.full((b, r, c // 32), 0xA5, dtype=torch.uint8, device="cuda"),
               "col_codes": torch.full((b, c, r * 3 // 4), 0xA5, dtype=torch.uint8, device="cuda"),
               "col_scales": torch.full((b, c, r // 32), 0xA5, dtype=torch.uint8, device="cuda")}
        for mode in MODES:
            got = mx.mx_quantize(x.cuda(), fmt, mode, "both", out=out)
            torch.cuda.synchronize()
            got = {k: v.cpu().numpy() for k, v in got.items()}
            assert_same(got, oracle_quant(x, fmt, mode, "both"), f"fp6 lines {(b, r, c, fmt, dt, mode)}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", FMTS)
def test_column_only_any_vector_width(mx, fmt, dt):
    """A column-only cast blocks no run along cols, so cols need only fill whole
    16-byte vectors (8 BF16 or 4 FP32): cols of 40, 36, 264 and 300 (a ragged
    last tile) with outputs that start as a sentinel and a guard band after
    each plane, batches, both scale rules."""
    g = torch.Generator().manual_seed(36)
    step = 8 if dt == "bf16" else 4
    bits = OFMT[fmt].bits
    for b, r, c in [(1, 64, 40), (2, 96, 8 * 37 if dt == "bf16" else 36), (1, 160, 264), (3, 32, 8 * 38 if dt == "bf16" else 300)]:
        assert c % step == 0
        x = torch.randn((b, r, c), generator=g) * torch.exp2(torch.randint(-8, 8, (b, 1, c), generator=g).float())
        x = x.to(torch.bfloat16) if dt == "bf16" else x
        for mode in MODES:
            nc, ns = b * c * r * bits // 8, b * c * (r // 32)
            cc = torch.full((nc + 64,), 0xA5, dtype=torch.uint8, device="cuda")
            cs = torch.full((ns + 64,), 0xA5, dtype=torch.uint8, device="cuda")
            got = mx.mx_quantize(x.cuda(), fmt, mode, "col", out={"col_codes": cc[:nc].view(b, c, r * bits // 8),
                                                                  "col_scales": cs[:ns].view(b, c, r // 32)})
            torch.cuda.synchronize()
            assert_same({k: v.cpu().numpy() for k, v in got.items()}, oracle_quant(x, fmt, mode, "col"),
                        f"col-only {(b, r, c)} {mode}")
            assert (cc[nc:].cpu() == 0xA5).all() and (cs[ns:].cpu() == 0xA5).all()


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", ["e4m3", "e2m1", "int8"])
def test_staggered_strip_order(mx, fmt, dt):
    """8192-row slices give column-plane pitches of 8 or 4 KiB and 64 tile rows,
    where the tiled kernel rotates each XCD strip's walk over the tile rows.
    Two slices (the rotation runs over both) and 288 columns (two tile columns,
    the second ragged). Outputs start as a sentinel, so a tile the walk skipped
    or visited twice with another tile's coordinates shows up."""
    g = torch.Generator().manual_seed(23)
    b, r, c = 2, 8192, 288
    x = torch.randn((b, r, c), generator=g) * torch.exp2(torch.randint(-6, 6, (b, r // 32, 1, 1), generator=g)
                                                        .float()).expand(b, r // 32, 32, 1).reshape(b, r, 1)
    x = x.to(torch.bfloat16) if dt == "bf16" else x
    bits = {"e4m3": 8, "e2m1": 4, "int8": 8}[fmt]
    for axis in ("both", "col"):
        out = {}
        if axis == "both":
            out["row_codes"] = torch.full((b, r, c * bits // 8), 0xA5, dtype=torch.uint8, device="cuda")
            out["row_scales"] = torch.full((b, r, c // 32), 0xA5, dtype=torch.uint8, device="cuda")
        out["col_codes"] = torch.full((b, c, r * bits // 8), 0xA5, dtype=torch.uint8, device="cuda")
        out["col_scales"] = torch.full((b, c, r // 32), 0xA5, dtype=torch.uint8, device="cuda")
        got = mx.mx_quantize(x.cuda(), fmt, "floor", axis, out=out)
        torch.cuda.synchronize()
        got = {k: v.cpu().numpy() for k, v in got.items()}
        assert_same(got, oracle_quant(x, fmt, "floor", axis), f"staggered {(b, r, c, fmt, dt, axis)}")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("fmt", NEW_FMTS)
def test_new_formats_workloads(mx, fmt, mode):
    """MXFP6 / MXINT8 on the workload tensors at small sizes: BF16 activations
    fused (several tiles, ragged tails), BF16 weights row-wise, FP32 gradients
    with specials column-wise and fused."""
    for shape in ((544, 416), (96, 4128), (32, 32)):
        check(mx, I.activations(*shape, seed=31), fmt, mode, "both", f"act{shape}")
    check(mx, I.weights(352, 288, seed=32), fmt, mode, "row", "weights")
    g = I.gradients(288, 352, seed=33)
    check(mx, g, fmt, mode, "col", "grads/col")
    check(mx, g, fmt, mode, "both", "grads/both")


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fmt", NEW_FMTS)
def test_new_formats_round_trip(mx, fmt, out_dtype):
    b, r, c = 2, 160, 288
    x = torch.stack([I.wide_range(i, r, c, seed=34) for i in range(b)])
    got = gpu_quant(mx, x, fmt, "floor", "both")
    exp = oracle_quant(x, fmt, "floor", "both")
    assert_same(got, exp, "wide")
    for plane, shp in (("row", (b, r, c)), ("col", (b, c, r))):
        y = mx.mx_dequantize(torch.from_numpy(got[f"{plane}_codes"]).cuda(),
                             torch.from_numpy(got[f"{plane}_scales"]).cuda(), fmt, shp, out_dtype)
        torch.cuda.synchronize()
        ref = O.dequantize(exp[f"{plane}_codes"], exp[f"{plane}_scales"], OFMT[fmt], out_dtype)
        yb = y.cpu().contiguous()
        yb = yb.view(torch.int16).numpy().view(np.uint16) if out_dtype == "bf16" else yb.numpy().view(np.uint32)
        assert np.array_equal(yb, ref), plane


# ---------------- dequantization ----------------

@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", FMTS)
def test_dequant_every_code_and_scale(mx, fmt, out_dtype):
    """Every element code under every scale code 0..255, each in its own block."""
    ncode = 1 << OFMT[fmt].bits
    codes = np.tile(np.arange(ncode, dtype=np.uint8), 256)
    scales = np.repeat(np.arange(256, dtype=np.uint8), ncode)
    blocks = np.zeros((codes.size, 32), dtype=np.uint8)
    blocks[:, :] = codes[:, None]                         # whole block holds the code
    packed = O.pack_codes(blocks, OFMT[fmt])
    sc = scales.reshape(-1, 1)
    y = mx.mx_dequantize(torch.from_numpy(np.ascontiguousarray(packed)).cuda(), torch.from_numpy(sc).cuda(),
                         fmt, (blocks.shape[0], 32), out_dtype)
    torch.cuda.synchronize()
    ref = O.dequantize(packed, sc, OFMT[fmt], out_dtype)
    yb = y.cpu()
    yb = yb.view(torch.int16).numpy().view(np.uint16) if out_dtype == "bf16" else yb.numpy().view(np.uint32)
    bad = np.argwhere(yb != ref)
    assert bad.size == 0, (bad[:3], blocks[bad[0][0], 0], sc[bad[0][0]], yb[tuple(bad[0])], ref[tuple(bad[0])])


# ---------------- large-tensor addressing ----------------
# (the workloads at full size are compared whole in test_gpu_full.py)

def slab_check(mx_out, x_slab_cpu, r0, fmt, mode, axis, batch_index=None):
    """Compare the rows r0..r0+n of the GPU planes with the oracle on that slab."""
    n = x_slab_cpu.shape[0]
    exp = oracle_quant(x_slab_cpu, fmt, mode, axis)
    bits = OFMT[fmt].bits
    for k, e in exp.items():
        t = mx_out[k] if batch_index is None else mx_out[k][batch_index]
        if k == "row_codes":
            g = t[r0:r0 + n]
        elif k == "row_scales":
            g = t[r0:r0 + n]
        elif k == "col_codes":
            g = t[:, r0 * bits // 8:(r0 + n) * bits // 8]
        else:
            g = t[:, r0 // 32:(r0 + n) // 32]
        g = g.cpu().numpy()
        bad = np.argwhere(g != e)
        assert bad.size == 0, (k, r0, bad[:3])


@pytest.mark.parametrize("fmt", ["e4m3", "e2m3"])
def test_tall_column_plane_addressing(mx, fmt):
    """4194432 x 256 BF16 (column-plane rows above 2^22 bytes apart): the slab
    that crosses row 2^22, every one of the 256 columns."""
    R, C = (1 << 22) + 128, 256
    x = I.activations(R, C, seed=35, device="cuda")
    out = mx.mx_quantize(x, fmt, "floor", "both")
    torch.cuda.synchronize()
    for r0 in ((1 << 22) - 128, R - 256):
        slab_check(out, x[r0:r0 + 256].cpu(), r0, fmt, "floor", "both")
    del out, x


@pytest.mark.parametrize("fmt,dt,rows", [("e4m3", "bf16", 160), ("e4m3", "bf16", 256), ("e2m1", "bf16", 256),
                                         ("e4m3", "f32", 256)])
def test_widest_row_plane_addressing(mx, fmt, dt, rows):
    """2^22 - 256 columns (the widest the ABI takes), so a tile's rows of the row plane
    span 128 x C bytes: every plane compared in the first and last 512 columns, all rows.
    160 rows: a ragged last tile and byte column scales; 256 rows: dword column scales."""
    R, C = rows, (1 << 22) - 256
    x = (I.activations(R, C, seed=41, device="cuda") if dt == "bf16"
         else I.gradients(R, C, seed=41, device="cuda"))
    out = mx.mx_quantize(x, fmt, "floor", "both")
    torch.cuda.synchronize()
    bits = OFMT[fmt].bits
    for c0 in (0, C - 512):
        exp = oracle_quant(x[:, c0:c0 + 512].cpu(), fmt, "floor", "both")
        got = {"row_codes": out["row_codes"][:, c0 * bits // 8:(c0 + 512) * bits // 8],
               "row_scales": out["row_scales"][:, c0 // 32:(c0 + 512) // 32],
               "col_codes": out["col_codes"][c0:c0 + 512], "col_scales": out["col_scales"][c0:c0 + 512]}
        assert_same({k: v.cpu().numpy() for k, v in got.items()}, exp, f"columns {c0}..+512")
    del out, x
