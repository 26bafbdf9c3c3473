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
