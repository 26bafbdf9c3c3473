"""Seeded random configurations through the C ABI, bit-exact against the CPU
oracle. Each case draws a shape within the entry point's rules (batches,
ragged last tiles, extents far from multiples of the tile, column counts that
are not multiples of 32 where a column-only cast allows them) and a random
format, axis, scale rule, rounding, block shape and input type, on data that
spans many binades and holds zeros and the occasional NaN or Inf. Outputs are
written into buffers that start as a sentinel, with a guard band after each
plane that must stay untouched. The cases are fixed by the seed, so a failure
names a reproducible configuration.
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
GUARD = 64
SENTINEL = 0xA5


def _data(rng, b, r, c, dt, specials):
    """Gaussian values times 2^k (k per row, in [-24, 24]), some exact zeros and,
    when asked, a few NaN / +-Inf."""
    x = rng.standard_normal((b, r, c)) * np.exp2(rng.integers(-24, 25, (b, r, 1)))
    x[rng.random((b, r, c)) < 0.02] = 0.0
    if specials:
        m = rng.random((b, r, c)) < 0.0005
        x[m] = rng.choice([np.nan, np.inf, -np.inf], size=int(m.sum()))
    t = torch.from_numpy(x.astype(np.float32))
    return t.to(torch.bfloat16) if dt == "bf16" else t


def _planes(shapes: dict, dtypes: dict | None = None):
    """Sentinel-filled buffers with a guard band; returns (views, buffers)."""
    views, bufs = {}, {}
    for k, shp in shapes.items():
        dt = (dtypes or {}).get(k, torch.uint8)
        n = int(np.prod(shp))
        if dt == torch.uint8:
            buf = torch.full((n + GUARD,), SENTINEL, dtype=torch.uint8, device="cuda")
        else:
            buf = torch.full((n + GUARD // 4,), float("nan"), dtype=dt, device="cuda")
        bufs[k], views[k] = buf, buf[:n].view(shp)
    return views, bufs


def _guards_intact(bufs: dict, shapes: dict):
    for k, buf in bufs.items():
        n = int(np.prod(shapes[k]))
        tail = buf[n:].cpu()
        if buf.dtype == torch.uint8:
            assert bool((tail == SENTINEL).all()), f"guard band after {k} overwritten"
        else:
            assert bool(torch.isnan(tail).all()), f"guard band after {k} overwritten"


def _same(got: dict, exp: dict, what: str):
    for k, e in exp.items():
        g = got[k]
        e = np.asarray(e)
        if e.dtype == np.float32:
            g, e = g.view(np.uint32), e.view(np.uint32)
        assert g.shape == e.shape, (what, k, g.shape, e.shape)
        bad = np.argwhere(g != e)
        if bad.size:
            idx = tuple(int(v) for v in bad[0])
            raise AssertionError(f"{what} {k}: {len(bad)} mismatches, first at {idx}: gpu={g[idx]:#x} "
                                 f"oracle={e[idx]:#x}")


def _mx_case(rng):
    fmt = str(rng.choice(list(OFMT)))
    mode = str(rng.choice(["floor", "roundup"]))
    axis = str(rng.choice(["row", "col", "both"]))
    rounding = str(rng.choice(["rne", "sr"]))
    block = str(rng.choice(["1x32", "32x32"], p=[0.75, 0.25]))
    dt = str(rng.choice(["bf16", "f32"]))
    b = int(rng.integers(1, 4))
    blocked_rows = axis != "row" or block == "32x32"
    blocked_cols = axis != "col" or block == "32x32"
    r = 32 * int(rng.integers(1, 13)) if blocked_rows else int(rng.integers(1, 400))
    if blocked_cols:
        c = 32 * int(rng.integers(1, 20))
    else:
        c = (8 if dt == "bf16" else 4) * int(rng.integers(1, 90))
    seed = int(rng.integers(0, 2 ** 63))
    return fmt, mode, axis, rounding, block, dt, b, r, c, seed


@pytest.mark.parametrize("case", range(160))
def test_random_mx_casts(mx, case):
    """mx_quantize / mx_quantize_ex with drawn options and shapes."""
    rng = np.random.default_rng(1000 + case)
    fmt, mode, axis, rounding, block, dt, b, r, c, seed = _mx_case(rng)
    what = f"case {case}: fmt={fmt} mode={mode} axis={axis} rounding={rounding} block={block} {dt} {(b, r, c)}"
    print(what, flush=True)
    x = _data(rng, b, r, c, dt, specials=bool(rng.random() < 0.3))
    bits = OFMT[fmt].bits
    two = block == "32x32"
    shapes = {}
    if axis != "col":
        shapes["row_codes"] = (b, r, c * bits // 8)
        shapes["row_scales"] = (b, r // 32, c // 32) if two else (b, r, c // 32)
    if axis != "row":
        shapes["col_codes"] = (b, c, r * bits // 8)
        shapes["col_scales"] = (b, c // 32, r // 32) if two else (b, c, r // 32)
    views, bufs = _planes(shapes)
    mx.mx_quantize(x.cuda(), fmt, mode, axis, out=views, rounding=rounding, seed=seed, block=block)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in views.items()}
    exp = O.quantize_ex(I.to_bits(x), dt, OFMT[fmt], OMODE[mode], OAXIS[axis], rounding, seed, block)
    _same(got, exp, what)
    _guards_intact(bufs, shapes)


@pytest.mark.parametrize("case", range(48))
def test_random_nvfp4_casts(mx, case):
    """mx_quantize_nvfp4 with drawn shapes, axes and input types; the global
    scale computed in the call or (one case in four) given by the caller."""
    rng = np.random.default_rng(2000 + case)
    axis = str(rng.choice(["row", "col", "both"]))
    dt = str(rng.choice(["bf16", "f32"]))
    b = int(rng.integers(1, 4))
    r = 16 * int(rng.integers(1, 25)) if axis != "row" else int(rng.integers(1, 300))
    c = 16 * int(rng.integers(1, 40))
    what = f"case {case}: nvfp4 axis={axis} {dt} {(b, r, c)}"
    print(what, flush=True)
    x = _data(rng, b, r, c, dt, specials=bool(rng.random() < 0.3))
    shapes = {"global_scale": (b,)}
    if axis != "col":
        shapes["row_codes"], shapes["row_scales"] = (b, r, c // 2), (b, r, c // 16)
    if axis != "row":
        shapes["col_codes"], shapes["col_scales"] = (b, c, r // 2), (b, c, r // 16)
    views, bufs = _planes(shapes, {"global_scale": torch.float32})
    given = None
    if rng.random() < 0.25:
        given = (np.abs(rng.standard_normal(b)) * np.exp2(rng.integers(-30, 10, b))).astype(np.float32)
        views["global_scale"].copy_(torch.from_numpy(given))
    mx.mx_quantize_nvfp4(x.cuda(), axis, global_scale=views["global_scale"] if given is not None else None,
                         out={k: v for k, v in views.items() if k != "global_scale"} | (
                             {"global_scale": views["global_scale"]} if given is None else {}))
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in views.items()}
    exp = O.nvfp4_quantize(I.to_bits(x), dt, OAXIS[axis], given)
    _same(got, exp, what)
    _guards_intact(bufs, shapes)


@pytest.mark.parametrize("case", range(32))
def test_random_requant(mx, case):
    """mx_requant_fp4_fp8 on a GPU-made MXFP4 plane of drawn shape and axis,
    and mx_quantize_fp4_fp8 (the one-pass step) on the same master weights."""
    rng = np.random.default_rng(3000 + case)
    axis = str(rng.choice(["row", "col", "both"]))
    mode = str(rng.choice(["floor", "roundup"]))
    dt = str(rng.choice(["bf16", "f32"]))
    b = int(rng.integers(1, 3))
    r = 16 * int(rng.integers(1, 30)) if axis != "row" else int(rng.integers(1, 500))
    c = 32 * int(rng.integers(1, 20))
    what = f"case {case}: requant axis={axis} mode={mode} {dt} {(b, r, c)}"
    print(what, flush=True)
    x = _data(rng, b, r, c, dt, specials=bool(rng.random() < 0.3))
    q = mx.mx_quantize(x.cuda(), "e2m1", mode, "row")
    out = mx.mx_requant_fp4_fp8(q["row_codes"], q["row_scales"], (b, r, c), axis)
    one = mx.mx_quantize_fp4_fp8(x.cuda(), mode, axis)
    torch.cuda.synchronize()
    codes, scales = q["row_codes"].cpu().numpy(), q["row_scales"].cpu().numpy()
    exp = O.requant_fp4_to_fp8(codes, scales)
    exp = {k: v for k, v in exp.items() if k in out}
    _same({k: v.cpu().numpy() for k, v in out.items()}, exp, what + " (requant)")
    ref_q = O.quantize(I.to_bits(x), dt, O.E2M1, OMODE[mode], O.ROW)
    exp1 = O.requant_fp4_to_fp8(ref_q["row_codes"], ref_q["row_scales"])
    exp1 = {k: v for k, v in exp1.items() if k in one}
    exp1["fp4_codes"], exp1["fp4_scales"] = ref_q["row_codes"], ref_q["row_scales"]
    _same({k: v.cpu().numpy() for k, v in one.items()}, exp1, what + " (one pass)")
