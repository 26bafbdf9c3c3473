"""Whole-tensor, bit-exact parity at the workloads' full sizes, in the launch
configuration the benchmark times: every code byte, scale byte and dequantized
bit of every plane against the CPU oracle ("MXFP4 と NVFP4 は何が違うのか調べてみた"
§2: 32-element blocks, E8M0 scales, round-to-nearest-even; §4: the floor and
round-up scale rules; §3 for NVFP4). The oracle runs over 512-row slabs in
forked worker processes (tests/whole_tensor.py); the GPU planes are copied to
host memory first.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import mx_inputs as I
import oracle as O
import whole_tensor as W

pytestmark = pytest.mark.gpu

OFMT = {"e4m3": O.E4M3, "e5m2": O.E5M2, "e2m1": O.E2M1, "e2m3": O.E2M3, "e3m2": O.E3M2, "int8": O.INT8}
OMODE = {"floor": O.FLOOR, "roundup": O.ROUNDUP}
OAXIS = {"row": O.ROW, "col": O.COL, "both": O.BOTH}


def mx_cols(fmt):
    return {"col_codes": Fraction(OFMT[fmt].bits, 8), "col_scales": Fraction(1, 32)}


def host(planes: dict, batched: bool) -> dict:
    return {k: (v.cpu().numpy() if batched else v.cpu().numpy()[None]) for k, v in planes.items()}


def bf16_bits(t):
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def quant_oracle(dtype, fmt, mode, axis):
    return lambda xs: O.quantize(xs, dtype, OFMT[fmt], OMODE[mode], OAXIS[axis])


def check_mx(mx, x, dtype, fmt, mode, axis, slabs):
    out = mx.mx_quantize(x, fmt, mode, axis)
    torch.cuda.synchronize()
    got = host(out, batched=False)
    xb = I.to_bits(x)[None]
    del out
    bad, n = W.compare(xb, quant_oracle(dtype, fmt, mode, axis), got, mx_cols(fmt))
    assert n == slabs
    assert not bad, bad[:5]


def test_whole_activations_fused_e4m3(mx):
    """16384x4096 BF16 activations (4 outlier columns x100), E4M3 row+col in one launch, floor."""
    check_mx(mx, I.activations(16384, 4096, seed=1, device="cuda"), "bf16", "e4m3", "floor", "both", 32)


@pytest.mark.parametrize("mode", ["floor", "roundup"])
def test_whole_weights_e2m1(mx, mode):
    """14336x4096 BF16 weights (per-row std log-uniform), E2M1 row-wise, both scale rules."""
    check_mx(mx, I.weights(14336, 4096, seed=2, device="cuda"), "bf16", "e2m1", mode, "row", 28)


def test_whole_gradients_e5m2_col(mx):
    """8192x8192 FP32 gradients (Student-t, zeros, +-Inf/NaN, zero blocks), E5M2 column-wise, round-up."""
    x = I.gradients(8192, 8192, seed=3, device="cuda")
    assert not bool(torch.isfinite(x).all())
    check_mx(mx, x, "f32", "e5m2", "roundup", "col", 16)


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2", "int8"])
def test_whole_activations_fused_new_formats(mx, fmt):
    """The fused cast of the 16384x4096 activations to MXFP6 and MXINT8."""
    check_mx(mx, I.activations(16384, 4096, seed=1, device="cuda"), "bf16", fmt, "floor", "both", 32)


@pytest.mark.parametrize("part", range(4))
def test_whole_wide_range_pipeline(mx, part):
    """64 x 4096x14336 BF16 (uniform x 2^k per 1x32 block, k in [-20, 20]): the
    fused E4M3 quantize of the whole batch in one launch and both planes
    dequantized to BF16, as the benchmark runs it. Tensors 16*part .. +15 are
    compared in full (codes, scales and both dequantized planes); the
    round-trip error bound of E4M3 under the floor rule is checked on them as
    well."""
    B, R, C = 64, 4096, 14336
    x = I.wide_range_batch(B, R, C, seed=4, device="cuda")
    out = mx.mx_quantize(x, "e4m3", "floor", "both")
    yr = mx.mx_dequantize(out["row_codes"], out["row_scales"], "e4m3", (B, R, C), "bf16")
    yc = mx.mx_dequantize(out["col_codes"], out["col_scales"], "e4m3", (B, C, R), "bf16")
    torch.cuda.synchronize()
    sl = slice(16 * part, 16 * part + 16)
    # extra: E4M3 with the floor rule puts a block's largest magnitude in [256, 512); elements
    # whose scaled magnitude is normal keep a relative error <= 2^-4, clipped ones lie in
    # [448, 512) * 2^e, and the rest are within half the subnormal step 2^-10 * 2^e
    for bi in range(sl.start, sl.stop):
        xf = x[bi].float()
        step = torch.exp2(out["row_scales"][bi].to(torch.int32).float() - 127 - 10).repeat_interleave(32, dim=1)
        err = (yr[bi].float() - xf).abs()
        assert bool(((err <= xf.abs() * 2.0 ** -4 + step) | (xf.abs() >= 448.0 * step * 1024)).all()), bi
    got = {k: v[sl].cpu().numpy() for k, v in out.items()}
    deq_got = {"row_deq": bf16_bits(yr[sl]), "col_deq": bf16_bits(yc[sl])}
    xb = I.to_bits(x[sl])
    del out, yr, yc, x

    def deq(exp):
        return {"row_deq": O.dequantize(exp["row_codes"][0], exp["row_scales"][0], O.E4M3, "bf16"),
                "col_deq": O.dequantize(exp["col_codes"][0], exp["col_scales"][0], O.E4M3, "bf16")}
    bad, n = W.compare(xb, quant_oracle("bf16", "e4m3", "floor", "both"), got, mx_cols("e4m3"), deq=deq,
                       deq_got=deq_got)
    assert n == 16 * 8
    assert not bad, bad[:5]


def test_whole_activations_nvfp4(mx):
    """16384x4096 BF16 activations, NVFP4 row+col with the global scale computed
    in the call: the global scale against the oracle's over the whole tensor,
    then every code and scale of both copies."""
    x = I.activations(16384, 4096, seed=1, device="cuda")
    out = mx.mx_quantize_nvfp4(x, "both")
    torch.cuda.synchronize()
    xb = I.to_bits(x)[None]
    g = O.nvfp4_global_scale(O.widen(xb, "bf16"))
    assert out["global_scale"].cpu().numpy().view(np.uint32)[0] == g.view(np.uint32)[0]
    got = host({k: v for k, v in out.items() if k != "global_scale"}, batched=False)
    del out, x
    bad, n = W.compare(xb, lambda xs: O.nvfp4_quantize(xs, "bf16", O.BOTH, g), got,
                       {"col_codes": Fraction(1, 2), "col_scales": Fraction(1, 16)})
    assert n == 32
    assert not bad, bad[:5]


# ---------------- the variants at full size ----------------

SR_SEED = 0x123456789ABCDEF0           # high key bits set


def test_whole_gradients_sr_e2m1_col(mx):
    """8192x8192 FP32 gradients to E2M1 columns with stochastic rounding (round-up
    scale rule): every code and scale, each slab drawing its bits at its flat
    offset in the tensor."""
    R = C = 8192
    x = I.gradients(R, C, seed=3, device="cuda")
    out = mx.mx_quantize(x, "e2m1", "roundup", "col", rounding="sr", seed=SR_SEED)
    torch.cuda.synchronize()
    got = host(out, batched=False)
    xb = I.to_bits(x)[None]
    del out, x

    def oracle(xs, bi, r0):
        return O.quantize_ex(xs, "f32", O.E2M1, O.ROUNDUP, O.COL, rounding=O.SR, seed=SR_SEED, first=r0 * C)
    bad, n = W.compare(xb, oracle, got, mx_cols("e2m1"), with_offset=True)
    assert n == 16
    assert not bad, bad[:5]


def test_whole_weights_2d_e2m1(mx):
    """14336x4096 BF16 weights to E2M1 with 32x32 blocks, both copies: every
    code and every scale of both scale grids."""
    x = I.weights(14336, 4096, seed=2, device="cuda")
    out = mx.mx_quantize(x, "e2m1", "floor", "both", block="32x32")
    torch.cuda.synchronize()
    got = host(out, batched=False)
    xb = I.to_bits(x)[None]
    del out, x
    bad, n = W.compare(xb, lambda xs: O.quantize_ex(xs, "bf16", O.E2M1, O.FLOOR, O.BOTH, block=O.BLOCK_32X32), got,
                       mx_cols("e2m1"), cut={"row_scales": ("row", Fraction(1, 32))})
    assert n == 28
    assert not bad, bad[:5]


FP8_CUT = {"e4m3": ("row", Fraction(1)), "block_scale": ("row", Fraction(1, 128)),
           "spread": ("row", Fraction(1, 128)), "e4m3_t": ("col", Fraction(1)),
           "block_scale_t": ("col", Fraction(1, 128)), "fp4_codes": ("row", Fraction(1)),
           "fp4_scales": ("row", Fraction(1))}


def fp8_host(out: dict) -> dict:
    """Planes to host memory, FP32 block scales as their bit patterns."""
    got = {k: v.cpu().numpy()[None] for k, v in out.items()}
    for k in ("block_scale", "block_scale_t"):
        if k in got:
            got[k] = got[k].view(np.uint32)
    return got


def fp8_bits(exp: dict) -> dict:
    exp = dict(exp)
    for k in ("block_scale", "block_scale_t"):
        exp[k] = np.asarray(exp[k], dtype=np.float32).view(np.uint32)
    return exp


def test_whole_fp4_in_fp8_requant(mx):
    """14336x4096 weights: the MXFP4 plane (floor rule) requantized to FP8 with
    128x128 block scales, as the benchmark runs it: every code of both copies,
    every block scale (as bits) and every spread. The slabs of 512 rows are 4
    block rows; the oracle gets the same MXFP4 plane the kernel read."""
    R, C = 14336, 4096
    w = I.weights(R, C, seed=2, device="cuda")
    q = mx.mx_quantize(w, "e2m1", "floor", "row")
    out = mx.mx_requant_fp4_fp8(q["row_codes"], q["row_scales"], (R, C), "both")
    torch.cuda.synchronize()
    got = fp8_host(out)
    src = np.concatenate([q["row_codes"].cpu().numpy(), q["row_scales"].cpu().numpy()], axis=1)[None]
    del out, q, w

    def oracle(xs):
        return fp8_bits(O.requant_fp4_to_fp8(xs[None, :, :C // 2], xs[None, :, C // 2:]))
    bad, n = W.compare(src, oracle, got, {}, cut=FP8_CUT)
    assert n == 28
    assert not bad, bad[:5]


def test_whole_qat_fp32_master(mx):
    """14336x4096 FP32 master weights through MXFP4 (floor rule) to both FP8
    copies in one pass: the MXFP4 plane, both FP8 copies, block scales and
    spreads, all against the oracle's quantize followed by its requantization."""
    R, C = 14336, 4096
    x = I.weights(R, C, seed=2, device="cuda").float()
    out = mx.mx_quantize_fp4_fp8(x, "floor", "both")
    torch.cuda.synchronize()
    got = fp8_host(out)
    xb = I.to_bits(x)[None]
    del out, x

    def oracle(xs):
        q = O.quantize(xs, "f32", O.E2M1, O.FLOOR, O.ROW)
        exp = fp8_bits(O.requant_fp4_to_fp8(q["row_codes"], q["row_scales"]))
        exp["fp4_codes"], exp["fp4_scales"] = q["row_codes"], q["row_scales"]
        return exp
    bad, n = W.compare(xb, oracle, got, {}, cut=FP8_CUT)
    assert n == 28
    assert not bad, bad[:5]
