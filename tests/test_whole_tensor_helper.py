"""The whole-tensor comparison helper (tests/whole_tensor.py) on the CPU: with
planes the oracle computes over the whole tensor it finds no mismatch, and a
single wrong byte planted in any plane (row, transposed column, dequantized,
another batch slice) is found in the right slab."""
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import whole_tensor as W


def _data(b, r, c, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((b, r, c)) * np.exp2(rng.integers(-6, 6, (b, r, 1)))).astype(np.float32)
    return x


@pytest.mark.parametrize("fmt", [O.E4M3, O.E2M1, O.E2M3])
def test_finds_nothing_then_every_planted_byte(fmt):
    b, r, c = 3, 96, 160
    x = _data(b, r, c, 1)
    whole = O.quantize(x, "f32", fmt, O.FLOOR, O.BOTH)
    col = {"col_codes": Fraction(fmt.bits, 8), "col_scales": Fraction(1, 32)}
    oracle = lambda xs: O.quantize(xs, "f32", fmt, O.FLOOR, O.BOTH)
    deq = lambda e: {"row_deq": O.dequantize(e["row_codes"][0], e["row_scales"][0], fmt, "f32"),
                     "col_deq": O.dequantize(e["col_codes"][0], e["col_scales"][0], fmt, "f32")}
    deq_got = {"row_deq": O.dequantize(whole["row_codes"], whole["row_scales"], fmt, "f32"),
               "col_deq": O.dequantize(whole["col_codes"], whole["col_scales"], fmt, "f32")}
    bad, n = W.compare(x, oracle, whole, col, slab=32, deq=deq, deq_got=deq_got)
    assert n == b * 3 and bad == []
    for k in ("row_codes", "row_scales", "col_codes", "col_scales", "row_deq", "col_deq"):
        got = {kk: v.copy() for kk, v in whole.items()}
        dg = {kk: v.copy() for kk, v in deq_got.items()}
        tgt = dg[k] if k.endswith("deq") else got[k]
        idx = (2,) + tuple(s - 1 for s in tgt.shape[1:])          # last element of the last slice
        tgt[idx] ^= 1
        bad, _ = W.compare(x, oracle, got, col, slab=32, deq=deq, deq_got=dg)
        assert len(bad) == 1 and bad[0][0] == k and bad[0][1] == 2 and bad[0][3] == 1, (k, bad)
        # the row planes put it in the last slab; the column planes in the slab of the last rows
        assert bad[0][2] == 64


def test_block_grids_and_slab_offsets():
    """32x32-block scale grids cut by ("row", 1/32) and ("col", 1/32), and an
    oracle that needs the slab's position (stochastic rounding draws follow the
    flat element index): the whole-tensor planes match slab by slab, and one
    planted byte in the row scale grid is found in its slab."""
    b, r, c = 2, 128, 96
    x = _data(b, r, c, 2)
    seed = 0x1234_5678_9ABC
    whole = [O.quantize_ex(x[i], "f32", O.E2M1, O.ROUNDUP, O.BOTH, rounding=O.SR, seed=seed, block=O.BLOCK_32X32,
                           first=i * r * c) for i in range(b)]
    got = {k: np.concatenate([w[k] for w in whole]) for k in whole[0]}
    col = {"col_codes": Fraction(1, 2), "col_scales": Fraction(1, 32)}
    cut = {"row_scales": ("row", Fraction(1, 32))}

    def oracle(xs, bi, r0):
        return O.quantize_ex(xs, "f32", O.E2M1, O.ROUNDUP, O.BOTH, rounding=O.SR, seed=seed, block=O.BLOCK_32X32,
                             first=(bi * r + r0) * c)
    bad, n = W.compare(x, oracle, got, col, slab=64, cut=cut, with_offset=True)
    assert n == b * 2 and bad == []
    got["row_scales"][1, 3, 0] ^= 1                          # tile row 3 of slice 1: rows 96..127
    bad, _ = W.compare(x, oracle, got, col, slab=64, cut=cut, with_offset=True)
    assert [(k, bi, r0) for k, bi, r0, *_ in bad] == [("row_scales", 1, 64)]
    # an oracle that ignored the offset would draw the wrong bits
    bad, _ = W.compare(x, lambda xs: O.quantize_ex(xs, "f32", O.E2M1, O.ROUNDUP, O.BOTH, rounding=O.SR, seed=seed,
                                                     block=O.BLOCK_32X32), got, col, slab=64, cut=cut)
    assert bad
