"""Bit-exact parity of the stochastic-rounding and 32x32-block casts (through
mx_quantize_ex / mx_dequantize_ex) with the CPU oracle."""
import numpy as np
import pytest
import torch

import mx_inputs as I
import oracle as O

pytestmark = pytest.mark.gpu

OFMT = {"e4m3": O.E4M3, "e5m2": O.E5M2, "e2m1": O.E2M1, "e2m3": O.E2M3, "e3m2": O.E3M2, "int8": O.INT8}
OMODE = {"floor": O.FLOOR, "roundup": O.ROUNDUP}
OAXIS = {"row": O.ROW, "col": O.COL, "both": O.BOTH}
FMTS = list(OFMT)
SEEDS = [0, 0x123456789ABCDEF0]


def gpu(mx, x, fmt, mode, axis, **kw):
    out = mx.mx_quantize(x.cuda().contiguous(), fmt, mode, axis, **kw)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def oracle(x, fmt, mode, axis, rounding="rne", seed=0, block="1x32", first=0):
    dt = "bf16" if x.dtype == torch.bfloat16 else "f32"
    out = O.quantize_ex(I.to_bits(x), dt, OFMT[fmt], OMODE[mode], OAXIS[axis], rounding, seed, block, first)
    if x.dim() == 2:
        out = {k: v[0] for k, v in out.items()}
    return out


def same(got, exp, what):
    assert set(got) == set(exp), (got.keys(), exp.keys())
    for k in exp:
        g, e = got[k], exp[k]
        assert g.shape == e.shape, (what, k, g.shape, e.shape)
        bad = np.argwhere(g != e)
        if bad.size:
            idx = tuple(bad[0])
            raise AssertionError(f"{what} {k}: {len(bad)} mismatches, first at {idx}: "
                                 f"gpu={g[idx]:#x} oracle={e[idx]:#x}")


def check(mx, x, fmt, mode, axis, what="", **kw):
    same(gpu(mx, x, fmt, mode, axis, **kw), oracle(x, fmt, mode, axis, **kw), what)


def pad_rows(t, mult=32):
    pad = (-t.shape[0]) % mult
    return torch.cat([t, torch.zeros((pad,) + tuple(t.shape[1:]), dtype=t.dtype)]) if pad else t


# ---------------- stochastic rounding ----------------

@pytest.mark.parametrize("fmt", FMTS)
def test_sr_bf16_sweep(mx, fmt):
    """Every BF16 pattern under every reachable scale, SR, rows (stream kernel)
    and fused row + column (tiled kernel)."""
    x = I.bf16_sweep(fmt)
    check(mx, x, fmt, "roundup", "row", "sweep/row", rounding="sr", seed=SEEDS[1])
    xc = pad_rows(x)[:4096].T.contiguous()
    check(mx, xc, fmt, "floor", "both", "sweep/both", rounding="sr", seed=SEEDS[0])


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["floor", "roundup"])
@pytest.mark.parametrize("fmt", FMTS)
def test_sr_edge_blocks(mx, fmt, mode, dt):
    x = pad_rows(I.fp32_edges(fmt) if dt == "f32" else I.bf16_edges(fmt))
    for seed in SEEDS:
        check(mx, x, fmt, mode, "row", "edges/row", rounding="sr", seed=seed)
        check(mx, x.T.contiguous(), fmt, mode, "both", "edges/both", rounding="sr", seed=seed)


@pytest.mark.parametrize("fmt", ["e2m1", "e5m2", "int8", "e3m2"])
def test_sr_workloads(mx, fmt):
    g = I.gradients(288, 352, seed=41)
    for axis in ("col", "both", "row"):
        check(mx, g, fmt, "roundup", axis, f"grads/{axis}", rounding="sr", seed=SEEDS[1])
    a = torch.stack([I.activations(160, 288, seed=42 + i) for i in range(2)])
    check(mx, a, fmt, "floor", "both", "act/both", rounding="sr", seed=7)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", FMTS)
def test_sr_column_only_ragged_cols(mx, fmt, dt):
    """Column-only casts with stochastic rounding and column counts that are not
    multiples of 32: FP32 (128-column tiles with 64-column waves) with 36, 100,
    300 and 132 columns, where every other row's Philox blocks start mid-lane-
    pair; BF16 with 40, 104, 264 and 136. Ragged last tiles, waves with no
    columns, batches, ragged tile rows, both scale rules and both seeds; FP32
    edge blocks; outputs start as a sentinel and a guard band follows each plane."""
    g = torch.Generator().manual_seed(44)
    bits = OFMT[fmt].bits
    cases = ([(1, 64, 36), (2, 96, 100), (1, 160, 300), (3, 32, 132)] if dt == "f32" else
             [(1, 64, 40), (2, 96, 104), (1, 160, 264), (3, 32, 136)])
    for i, (b, r, c) in enumerate(cases):
        x = torch.randn((b, r, c), generator=g) * torch.exp2(torch.randint(-10, 10, (b, 1, c), generator=g).float())
        x = x.to(torch.bfloat16) if dt == "bf16" else x
        mode = ("floor", "roundup")[i % 2]
        seed = SEEDS[i % 2]
        nc, ns = b * c * r * bits // 8, b * c * (r // 32)
        cc = torch.full((nc + 64,), 0xA5, dtype=torch.uint8, device="cuda")
        cs = torch.full((ns + 64,), 0xA5, dtype=torch.uint8, device="cuda")
        got = mx.mx_quantize(x.cuda(), fmt, mode, "col", rounding="sr", seed=seed,
                             out={"col_codes": cc[:nc].view(b, c, r * bits // 8), "col_scales": cs[:ns].view(b, c, r // 32)})
        torch.cuda.synchronize()
        same({k: v.cpu().numpy() for k, v in got.items()}, oracle(x, fmt, mode, "col", rounding="sr", seed=seed),
             f"sr col-only {(b, r, c)}")
        assert (cc[nc:].cpu() == 0xA5).all() and (cs[ns:].cpu() == 0xA5).all()
    e = pad_rows(I.fp32_edges(fmt) if dt == "f32" else I.bf16_edges(fmt))
    for mode in ("floor", "roundup"):
        check(mx, e, fmt, mode, "col", "edges/col", rounding="sr", seed=SEEDS[1])


def test_sr_draws_depend_on_seed_only(mx):
    x = I.gradients(256, 256, seed=43).cuda()
    a = mx.mx_quantize(x, "e2m1", "roundup", "col", rounding="sr", seed=5)
    b = mx.mx_quantize(x, "e2m1", "roundup", "col", rounding="sr", seed=5)
    c = mx.mx_quantize(x, "e2m1", "roundup", "col", rounding="sr", seed=6)
    torch.cuda.synchronize()
    assert torch.equal(a["col_codes"], b["col_codes"])
    assert not torch.equal(a["col_codes"], c["col_codes"])
    assert torch.equal(a["col_scales"], c["col_scales"])


# ---------------- 32x32 blocks ----------------

@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", FMTS)
def test_2d_edge_blocks(mx, fmt, dt):
    x = pad_rows(I.fp32_edges(fmt) if dt == "f32" else I.bf16_edges(fmt))
    for mode in ("floor", "roundup"):
        check(mx, x, fmt, mode, "row", "edges/row", block="32x32")
        check(mx, x.T.contiguous(), fmt, mode, "both", "edges/both", block="32x32")


@pytest.mark.parametrize("fmt", FMTS)
def test_2d_workloads(mx, fmt):
    w = I.weights(352, 288, seed=44)
    for axis in ("row", "col", "both"):
        check(mx, w, fmt, "floor", axis, f"weights/{axis}", block="32x32")
    check(mx, I.gradients(288, 352, seed=45), fmt, "roundup", "both", "grads", block="32x32")
    a = torch.stack([I.activations(96, 224, seed=46 + i) for i in range(3)])
    check(mx, a, fmt, "roundup", "both", "act", block="32x32")
    check(mx, I.activations(32, 4128, seed=49), fmt, "floor", "both", "wide", block="32x32")


@pytest.mark.parametrize("fmt", ["e2m1", "e4m3", "int8"])
def test_2d_with_sr(mx, fmt):
    w = I.weights(352, 288, seed=50)
    check(mx, w, fmt, "floor", "both", "weights", block="32x32", rounding="sr", seed=SEEDS[1])
    g = I.gradients(224, 160, seed=51)
    check(mx, g, fmt, "roundup", "row", "grads", block="32x32", rounding="sr", seed=3)


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", FMTS)
def test_2d_dequant(mx, fmt, out_dtype):
    b, r, c = 2, 160, 288
    x = torch.stack([I.wide_range(i, r, c, seed=52) for i in range(b)])
    got = gpu(mx, x, fmt, "floor", "both", block="32x32")
    exp = oracle(x, fmt, "floor", "both", block="32x32")
    same(got, exp, "quant")
    for plane, shp in (("row", (b, r, c)), ("col", (b, c, r))):
        y = mx.mx_dequantize(torch.from_numpy(got[f"{plane}_codes"]).cuda(),
                             torch.from_numpy(got[f"{plane}_scales"]).cuda(), fmt, shp, out_dtype, block="32x32")
        torch.cuda.synchronize()
        ref = O.dequantize_2d(exp[f"{plane}_codes"], exp[f"{plane}_scales"], OFMT[fmt], out_dtype)
        yb = y.cpu().contiguous()
        yb = yb.view(torch.int16).numpy().view(np.uint16) if out_dtype == "bf16" else yb.numpy().view(np.uint32)
        assert np.array_equal(yb, ref), plane


def test_2d_dequant_every_code_and_scale(mx):
    """32x32 tiles, each holding one code under one scale, for every E4M3 code
    and every scale code, so the tile indexing of the scale grid is exercised."""
    codes = np.repeat(np.arange(256, dtype=np.uint8), 32 * 32).reshape(256, 32, 32)
    scales = np.random.default_rng(3).integers(0, 256, 256, dtype=np.uint8)
    x = codes.reshape(16, 16, 32, 32).transpose(0, 2, 1, 3).reshape(512, 512)
    s2 = scales.reshape(16, 16)
    y = mx.mx_dequantize(torch.from_numpy(np.ascontiguousarray(x)).cuda(), torch.from_numpy(s2).cuda(), "e4m3",
                         (1, 512, 512), "f32", block="32x32")
    torch.cuda.synchronize()
    ref = O.dequantize_2d(x[None], s2[None], O.E4M3, "f32")[0]
    assert np.array_equal(y.cpu().numpy().reshape(512, 512).view(np.uint32), ref)

# (the 8192x8192 stochastic-rounding cast and the 14336x4096 32x32-block cast
# are compared whole in test_gpu_full.py)
