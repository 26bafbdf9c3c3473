"""Bit-exact parity of the NVFP4 cast and dequantization (mx_quantize_nvfp4,
mx_dequantize_nvfp4) with the CPU oracle."""
import numpy as np
import pytest
import torch

import mx_inputs as I
import oracle as O

pytestmark = pytest.mark.gpu

OAXIS = {"row": O.ROW, "col": O.COL, "both": O.BOTH}


def gpu(mx, x, axis, **kw):
    out = mx.mx_quantize_nvfp4(x.cuda().contiguous(), axis, **kw)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def oracle(x, axis, global_scale=None):
    dt = "bf16" if x.dtype == torch.bfloat16 else "f32"
    out = O.nvfp4_quantize(I.to_bits(x), dt, OAXIS[axis], global_scale)
    if x.dim() == 2:
        out = {k: (v if k == "global_scale" else v[0]) for k, v in out.items()}
    return out


def same(got, exp, what):
    assert set(got) == set(exp), (got.keys(), exp.keys())
    for k in exp:
        g, e = got[k], exp[k]
        if k == "global_scale":
            g, e = g.view(np.uint32), np.asarray(e, np.float32).view(np.uint32)
        assert g.shape == e.shape, (what, k, g.shape, e.shape)
        bad = np.argwhere(g != e)
        if bad.size:
            idx = tuple(bad[0])
            raise AssertionError(f"{what} {k}: {len(bad)} mismatches, first at {idx}: "
                                 f"gpu={g[idx]:#x} oracle={e[idx]:#x}")


def check(mx, x, axis, what=""):
    same(gpu(mx, x, axis), oracle(x, axis), what)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("axis", ["row", "col", "both"])
def test_shapes_and_ragged_tails(mx, axis, dt):
    g = torch.Generator().manual_seed(61)
    for b, r, c in [(1, 16, 16), (2, 48, 80), (1, 128, 256), (3, 144, 272), (1, 272, 4112), (2, 80, 64)]:
        x = torch.randn((b, r, c), generator=g) * torch.exp2(torch.randint(-10, 10, (b, r, 1), generator=g).float())
        x = x.to(torch.bfloat16) if dt == "bf16" else x
        check(mx, x, axis, f"{(b, r, c)}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_edges_specials_and_zero(mx, dt):
    x = I.fp32_edges("e2m1")
    x = x.to(torch.bfloat16) if dt == "bf16" else x
    x = x[: (x.shape[0] // 16) * 16]
    check(mx, x, "row", "edges/row")
    check(mx, x.T.contiguous(), "both", "edges/both")
    check(mx, torch.zeros((2, 32, 64), dtype=x.dtype), "both", "zeros")
    grads = I.gradients(144, 96, seed=62)
    assert not torch.isfinite(grads).all()
    check(mx, grads, "both", "grads")


def test_wide_dynamic_range(mx):
    """Blocks far below the tensor max fall under UE4M3's range and store zeros."""
    x = torch.stack([I.wide_range(i, 96, 320, seed=63) for i in range(2)])
    check(mx, x, "both", "wide")
    check(mx, I.weights(352, 288, seed=64), "both", "weights")


def test_given_global_scale(mx):
    x = I.activations(160, 288, seed=65)
    gs = torch.tensor([0.0371], dtype=torch.float32)
    out = mx.mx_quantize_nvfp4(x.cuda(), "both", global_scale=gs.cuda())
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in out.items()}
    same(got, oracle(x, "both", gs.numpy()), "given")


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_dequant_every_code_and_scale(mx, out_dtype):
    codes = np.tile(np.arange(256, dtype=np.uint8), 512).reshape(1, 2048, 64)   # 128 elements per row
    rng = np.random.default_rng(66)
    scales = rng.integers(0, 256, (1, 2048, 8), dtype=np.uint8)
    scales[0, :128, 0] = np.arange(128)                         # every UE4M3 code, and 0x80.. too
    scales[0, 128:256, 0] = np.arange(128, 256)
    for gval in (1.0, 3.1e-5, 7.7e30, 1e-38):
        gs = np.array([gval], np.float32)
        y = mx.mx_dequantize_nvfp4(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                                   torch.from_numpy(gs).cuda(), (1, 2048, 128), out_dtype)
        torch.cuda.synchronize()
        ref = O.nvfp4_dequantize(codes, scales, gs, out_dtype)
        yb = y.cpu()
        yb = yb.view(torch.int16).numpy().view(np.uint16) if out_dtype == "bf16" else yb.numpy().view(np.uint32)
        bad = np.argwhere(yb != ref)
        assert bad.size == 0, (gval, bad[:3])


def test_round_trip_through_both_calls(mx):
    x = I.activations(256, 512, seed=67)
    out = mx.mx_quantize_nvfp4(x.cuda(), "both")
    yr = mx.mx_dequantize_nvfp4(out["row_codes"], out["row_scales"], out["global_scale"], (1, 256, 512), "bf16")
    yc = mx.mx_dequantize_nvfp4(out["col_codes"], out["col_scales"], out["global_scale"], (1, 512, 256), "f32")
    torch.cuda.synchronize()
    exp = oracle(x, "both")
    same({k: v.cpu().numpy() for k, v in out.items()}, exp, "quant")
    rr = O.nvfp4_dequantize(exp["row_codes"][None], exp["row_scales"][None], exp["global_scale"], "bf16")[0]
    rc = O.nvfp4_dequantize(exp["col_codes"][None], exp["col_scales"][None], exp["global_scale"], "f32")[0]
    got_r = yr.cpu().view(torch.int16).numpy().view(np.uint16)[0]
    bad = np.argwhere(got_r != rr)
    assert bad.size == 0, (len(bad), bad[:4], got_r[tuple(bad[0])], rr[tuple(bad[0])])
    got_c = yc.cpu().numpy().view(np.uint32)[0]
    bad = np.argwhere(got_c != rc)
    assert bad.size == 0, (len(bad), bad[:4], got_c[tuple(bad[0])], rc[tuple(bad[0])])


def _midpoint_blocks(A, seed):
    """FP32 [R][256]: one element of magnitude A (so the tensor's global scale is
    fp32(A / 2688)); every other 16-element block has its max within +-20 ulps
    of a value whose scaled t sits on an E4M3 value or rounding midpoint."""
    rng = np.random.default_rng(seed)
    g = np.float32(A) / np.float32(2688)
    vals = O.value_table(O.E4M3)[:127]
    targets = np.concatenate([(vals[:-1] + vals[1:]) / 2, vals[1:], [464.0]])
    n = len(targets) * 41
    a = (np.repeat(targets, 41) * 6.0 * np.float64(g)).astype(np.float32)
    a = (a.view(np.int32) + np.tile(np.arange(-20, 21, dtype=np.int32), len(targets))).view(np.float32)
    a = np.minimum(a, np.float32(A))
    blocks = (rng.random((n, 16)) * 0.9).astype(np.float32) * a[:, None]
    blocks[np.arange(n), rng.integers(0, 16, n)] = a * np.where(rng.random(n) < 0.5, -1, 1).astype(np.float32)
    blocks = np.concatenate([blocks, np.full((1, 16), A, np.float32)])
    pad = (-len(blocks)) % 16
    blocks = np.concatenate([blocks, np.zeros((pad, 16), np.float32)])
    return torch.from_numpy(blocks.reshape(-1, 256))


@pytest.mark.parametrize("A", [1000.0, 2688.0, 3.0e-30, 2.0 ** -110, 1.5e30])
def test_block_codes_near_midpoints(mx, A):
    """Block maxima next to every UE4M3 rounding boundary: the fast block-code
    estimate must fall back wherever it cannot decide, and agree elsewhere."""
    x = _midpoint_blocks(A, seed=67)
    check(mx, x, "row", "mid/row")
    xr = x[: (x.shape[0] // 16) * 16]
    check(mx, xr.T.contiguous(), "both", "mid/both")


def test_tiny_fp32_blocks(mx):
    """FP32 blocks below 2^-120 under a normal global scale: their scaled maxima
    still reach UE4M3 subnormals, and they take the exact two-division path."""
    rng = np.random.default_rng(69)
    e = rng.uniform(-149, -117, (64, 16, 1))
    x = (rng.standard_normal((64, 16, 16)) * np.exp2(e)).astype(np.float32).reshape(64, 256)
    x[0, 0] = np.float32(2.0 ** -110)
    check(mx, torch.from_numpy(x), "both", "tiny")


@pytest.mark.parametrize("gval", [0.0, 1e-38, 2.0 ** -125, 2.0 ** -126, 3.3e-30, 0.0371, 2.0 ** 100, 2.0 ** 101, 1e37])
def test_given_global_scale_extremes(mx, gval):
    """Caller-given global scales inside and outside the range where the block
    code is estimated, over blocks spanning many binades."""
    rng = np.random.default_rng(68)
    e = rng.integers(-149, 128, (96, 1)).astype(np.float64)
    x = (rng.standard_normal((96, 256)) * np.exp2(np.clip(e, -149, 126))).astype(np.float32)
    x = torch.from_numpy(x)
    gs = torch.tensor([gval], dtype=torch.float32)
    out = mx.mx_quantize_nvfp4(x.cuda(), "both", global_scale=gs.cuda())
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in out.items()}
    same(got, oracle(x, "both", gs.numpy()), f"given {gval}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_row_scale_words(mx, dt):
    """With both copies, cols % 256 == 0 and a 16-byte-aligned row-scale plane,
    a tile row's 16 row-scale bytes are stored as one word after the barrier:
    batches, ragged tile rows, sentinel-filled outputs, and a plane offset by
    4 bytes that must take the per-wave stores instead."""
    g = torch.Generator().manual_seed(33)
    for b, r, c in [(2, 160, 512), (1, 4128, 256), (3, 64, 768)]:
        x = torch.randn((b, r, c), generator=g) * torch.exp2(torch.randint(-6, 6, (b, r, 1), generator=g).float())
        x = x.to(torch.bfloat16) if dt == "bf16" else x
        exp = oracle(x, "both")
        n = b * r * (c // 16)
        for shift in (0, 4):
            rs = torch.full((n + 16,), 0xA5, dtype=torch.uint8, device="cuda")
            out = {"row_codes": torch.full((b, r, c // 2), 0xA5, dtype=torch.uint8, device="cuda"),
                   "row_scales": rs[shift:shift + n].view(b, r, c // 16),
                   "col_codes": torch.full((b, c, r // 2), 0xA5, dtype=torch.uint8, device="cuda"),
                   "col_scales": torch.full((b, c, r // 16), 0xA5, dtype=torch.uint8, device="cuda")}
            got = mx.mx_quantize_nvfp4(x.cuda(), "both", out=out)
            torch.cuda.synchronize()
            same({k: v.cpu().numpy() for k, v in got.items()}, exp, f"nvfp4 row scale words {(b, r, c, dt, shift)}")
            guard = rs.cpu().numpy()
            assert (guard[:shift] == 0xA5).all() and (guard[shift + n:] == 0xA5).all()


def _e2m1_midpoint_blocks(g, seed):
    """FP32 blocks, for every UE4M3 block code s: a block max of fp32(6 s g)
    and elements within 0, 1, 2, 5 and 40 FP32 ulps of every E2M1 value and
    every midpoint between them, times s g, with random signs."""
    rng = np.random.default_rng(seed)
    vals = O.value_table(O.E4M3)[1:0x7F]
    pts = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    offs = np.array([0, 1, -1, 2, -2, 5, -5, 40, -40], np.int32)
    blocks = []
    for s in vals:
        top = np.float32(6.0 * s * np.float64(g))
        if not np.isfinite(top) or top == 0:
            continue
        el = (np.repeat(pts, len(offs)) * s * np.float64(g)).astype(np.float32)
        el = (el.view(np.int32) + np.tile(offs, len(pts))).view(np.float32)
        el = el[np.isfinite(el) & (el > 0) & (el <= top)]
        el = el * np.where(rng.random(el.size) < 0.5, -1, 1).astype(np.float32)
        pad = (-el.size) % 15
        el = np.concatenate([el, np.zeros(pad, np.float32)]).reshape(-1, 15)
        blocks.append(np.concatenate([np.full((el.shape[0], 1), top, np.float32), el], axis=1))
    b = np.concatenate(blocks)
    b = np.concatenate([b, np.zeros(((-len(b)) % 16, 16), np.float32)])
    return torch.from_numpy(b.reshape(-1, 256))


@pytest.mark.parametrize("gval", [1.0, 1.0 / 3.0, 0.0123, 2.0 ** -10, 2.0 ** -140, 3 * 2.0 ** -147])
def test_element_codes_near_e2m1_midpoints(mx, gval):
    """Elements next to every E2M1 rounding boundary under every block code:
    the hardware rounding of x * r_b must give way to the exact comparison
    wherever the two can differ (also where s_b * g is not a normal FP32)."""
    gs = np.array([gval], np.float32)
    x = _e2m1_midpoint_blocks(gs[0], seed=70)
    x = torch.cat([x, torch.zeros(((-x.shape[0]) % 16, 256), dtype=x.dtype)])     # rows % 16 for the column copy
    for xx, axis in ((x, "row"), (x.T.contiguous(), "both")):
        out = mx.mx_quantize_nvfp4(xx.cuda(), axis, global_scale=torch.from_numpy(gs).cuda())
        torch.cuda.synchronize()
        same({k: v.cpu().numpy() for k, v in out.items()}, oracle(xx, axis, gs), f"e2m1 mid {gval} {axis}")
    xb = x.to(torch.bfloat16)
    check(mx, xb, "both", f"e2m1 mid bf16 {gval}")


def test_midpoint_ties_with_computed_global_scale(mx):
    """A = 2688 gives g = 1 and a block max of 18 the block scale 3: 0.75,
    2.25, 7.5 and 15 sit exactly on E2M1 midpoints and go to the even codes."""
    x = torch.zeros((32, 256), dtype=torch.float32)
    x[0, 0] = 2688.0
    x[1, :7] = torch.tensor([18.0, 0.75, -0.75, 2.25, 7.5, 15.0, 4.5])
    for dt in (torch.float32, torch.bfloat16):
        check(mx, x.to(dt), "both", f"ties {dt}")
    out = mx.mx_quantize_nvfp4(x.cuda(), "row")
    torch.cuda.synchronize()
    assert out["row_scales"][1, 0].item() == 0x44
    assert out["row_codes"][1, :4].cpu().tolist() == [0x07, 0x28, 0x64, 0x03]


@pytest.mark.parametrize("gval", [-1.0, float("inf"), float("nan")])
def test_unusable_given_global_scale(mx, gval):
    """A given g that is not a finite positive number: scale 0 and codes 0 for
    every finite block, 0x7F for blocks holding NaN or Inf."""
    x = I.gradients(64, 96, seed=71)
    gs = torch.tensor([gval], dtype=torch.float32)
    out = mx.mx_quantize_nvfp4(x.cuda(), "both", global_scale=gs.cuda())
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in out.items()}
    exp = oracle(x, "both", gs.numpy())
    assert (exp["row_codes"] == 0).all() and (exp["row_scales"] != 0x7F).sum() == (exp["row_scales"] == 0).sum()
    same(got, exp, f"unusable g {gval}")
