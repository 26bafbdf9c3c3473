"""Whole-tensor parity: the CPU oracle over row slabs in forked worker processes.

Test infrastructure (imported by the GPU parity tests). The GPU's planes are
first copied to host memory; the pool is forked after that, so the workers
share those arrays copy-on-write and never touch the GPU. Each worker runs the
oracle on one slab of rows of one batch slice and compares every code and
scale byte (and, where asked, every dequantized bit) of the slab with the
GPU's planes:
  * row planes [B][R][...]: rows r0 .. r0+n;
  * column planes [B][C][...] (stored transposed): the slab's part of each
    column-plane row, bytes r0 * f .. (r0+n) * f for a plane with f bytes per
    input row (codes: bits / 8; MX scales: 1/32; NVFP4 scales: 1/16);
  * other planes as `cut` names them: ("row", f) takes plane rows r0 * f ..
    (r0+n) * f (a 32x32-block scale grid: f = 1/32), ("col", f) as above.
"""
from __future__ import annotations

import multiprocessing as mp
import os
from fractions import Fraction

import numpy as np

_JOB = None          # the job of the pool being forked (read by the workers)


def workers() -> int:
    """Worker processes: the machine's CPU share for one GPU is 16 processes; the
    parent (which holds the GPU) is one of them."""
    return max(1, min(15, os.cpu_count() or 1))


def _cut(plane: str, arr, r0: int, n: int, col_factor: dict, cut: dict | None = None):
    if cut and plane in cut:
        side, f = cut[plane]
    elif plane.startswith("row"):
        side, f = "row", Fraction(1)
    else:
        side, f = "col", col_factor[plane]
    a, b = int(r0 * f), int((r0 + n) * f)
    assert a == r0 * f and b == (r0 + n) * f, (plane, r0, n)
    return arr[a:b] if side == "row" else arr[:, a:b]


def _slab(task):
    bi, r0, n = task
    J = _JOB
    xs = J["x"][bi, r0:r0 + n]
    exp = J["oracle"](xs, bi, r0) if J["with_offset"] else J["oracle"](xs)
    bad = []
    for k, e in exp.items():
        if k not in J["got"]:
            continue
        g = _cut(k, J["got"][k][bi], r0, n, J["col_factor"], J["cut"])
        e = np.asarray(e)[0]
        if g.shape != e.shape or not np.array_equal(g, e):
            idx = np.argwhere(g != e) if g.shape == e.shape else np.zeros((1, 2), int)
            bad.append((k, bi, r0, int(len(idx)), tuple(int(v) for v in idx[0]), "shape" if g.shape != e.shape else ""))
    if J["deq"] is not None:
        for k, e in J["deq"](exp).items():
            g = _cut(k, J["deq_got"][k][bi], r0, n, {k: Fraction(1)})
            if not np.array_equal(g, e):
                idx = np.argwhere(g != e)
                bad.append((k, bi, r0, int(len(idx)), tuple(int(v) for v in idx[0]), "dequantized"))
    return bad


def compare(x_bits, oracle, got: dict, col_factor: dict, slab: int = 512, batches=None, deq=None,
            deq_got: dict | None = None, cut: dict | None = None, with_offset: bool = False):
    """Compare the GPU planes `got` (name -> numpy [B][...]) with `oracle`
    (a function of one slab x_bits[b, r0:r0+n] -> dict of planes with a
    leading batch axis of 1; called as oracle(slab, b, r0) when with_offset)
    over every slab of the listed batch slices. `deq(exp)` may return
    dequantized planes of the slab ("row_deq" [n][C], "col_deq" [C][n]) to
    compare with deq_got. Returns (mismatches, slabs)."""
    global _JOB
    B, R = x_bits.shape[0], x_bits.shape[1]
    assert slab % 32 == 0
    batches = range(B) if batches is None else batches
    tasks = [(b, r0, min(slab, R - r0)) for b in batches for r0 in range(0, R, slab)]
    _JOB = {"x": x_bits, "oracle": oracle, "got": got, "col_factor": col_factor, "deq": deq, "deq_got": deq_got,
            "cut": cut, "with_offset": with_offset}
    try:
        with mp.get_context("fork").Pool(workers()) as pool:
            results = pool.map(_slab, tasks, chunksize=1)
    finally:
        _JOB = None
    return [r for res in results for r in res], len(tasks)
