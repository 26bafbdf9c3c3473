"""Throughput of the fused row+column MXFP8 cast on one MI355X.

Workload (default): a 16384x4096 BF16 activation tensor (N(0,1) with 4
outlier columns x100, seeded, synthetic), quantized to MXFP8 E4M3 with the OCP
floor scale rule, row-wise and column-wise (transposed) copies emitted by one
kernel. One step = one such cast over one tensor, inputs already resident in
HBM. Eight input/output buffer sets rotate (2.2 GB), so nothing a step reads or
writes is still in the 256 MB last-level cache when that set comes round again.
Before the W warm-up steps the GPU runs the same step for at least 150 ms,
untimed, so the timed steps run at steady clocks. --workload selects the other
workloads (the other tensor configurations and the format variants), measured
the same way.

Prints one JSON line. `value` is GB/s of algorithmic traffic (each input byte
read once, each code and scale byte written once: 272,629,760 B per step for
the default). `roofline` compares the dominant kernel's rate (its algorithmic
bytes per launch over its average launch time, from HIP events on the launch
stream) with MI355X's 8 TB/s HBM peak; `traffic` carries the HBM bytes per
launch that rocprofv3 counters measured for the same kernel source
(profiles/<workload>_counters.txt), or null if the kernel changed since.
`cpu_baseline` times the CPU oracle over the same workload in forked worker
processes (the machine's CPU share for one GPU, 16 processes), `cpu_baseline_single`
on one core over a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# VALU issue peak of MI355X, non-packed: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
VALU_PEAK_T_LANE_OPS = 256 * 4 * 16 * 2.4e9 / 1e12          # 39.32 T lane-ops/s
CPU_PROCS = 16                                              # the machine's CPU share for one GPU
CSRC = "microscaling_block_quantized_amd/csrc/"
COMMON_SOURCES = [CSRC + f for f in ("mx_api.cpp", "mx_grid.cpp", "mx_kernels.h", "mx_enums.h", "mx_device.h")]
CAST_SOURCES = COMMON_SOURCES + [CSRC + f for f in ("mx_cast_impl.h", "mx_sr.h", "mx_cast.hip")]
COPY_KERNEL = "__amd_rocclr_copyBuffer"
LIB_COPY_KERNEL = "copy_nt_kernel"
CODE_BITS = {"e4m3": 8, "e5m2": 8, "e2m1": 4, "e2m3": 6, "e3m2": 6, "int8": 8}


def copy_bytes(alg_bytes: int) -> int:
    """Bytes each way of the ceiling copy: the workload's read+write byte count,
    but at least 256 MiB each way so four buffers exceed the 256 MB cache."""
    return min(max(alg_bytes // 2, 1 << 28), 1 << 31)


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

def _planes(dev, b, r, c, fmt, axis, block="1x32"):
    import torch
    bits = CODE_BITS[fmt]
    two = block == "32x32"
    out = {}
    if axis in ("row", "both"):
        out["row_codes"] = torch.empty((b, r, c * bits // 8), dtype=torch.uint8, device=dev)
        out["row_scales"] = torch.empty((b, r // 32, c // 32) if two else (b, r, c // 32), dtype=torch.uint8,
                                        device=dev)
    if axis in ("col", "both"):
        out["col_codes"] = torch.empty((b, c, r * bits // 8), dtype=torch.uint8, device=dev)
        out["col_scales"] = torch.empty((b, c // 32, r // 32) if two else (b, c, r // 32), dtype=torch.uint8,
                                        device=dev)
    return out


def _gen(name):
    def g(dev, i):
        import mx_inputs as I
        if name == "activations":
            return I.activations(16384, 4096, seed=1 + i, device=dev)
        if name == "weights":
            return I.weights(14336, 4096, seed=2 + 100 * i, device=dev)
        if name == "gradients":
            return I.gradients(8192, 8192, seed=3 + 100 * i, device=dev)
        raise KeyError(name)
    return g


def _cast_kernel_name(bf16, fmt, mode, axis, rounding, block):
    f = {"e4m3": 0, "e5m2": 1, "e2m1": 2, "e2m3": 3, "e3m2": 4, "int8": 5}[fmt]
    m = {"floor": 0, "roundup": 1}[mode]
    b = "true" if bf16 else "false"
    rd = 1 if rounding == "sr" else 0
    if axis == "row" and block == "1x32":
        return f"mx_cast_rows_kernel<{b}, {f}, {m}, {rd}>"
    ax = {"row": 1, "col": 2, "both": 3}[axis]
    return f"mx_cast_kernel<{b}, {f}, {m}, {ax}, {rd}, {'true' if block == '32x32' else 'false'}>"


def _mx_oracle_slab(dtype, fmt, mode, axis, rounding="rne", block="1x32"):
    """The oracle's quantization of rows r0 .. r0+n of a [B][R][C] tensor."""
    def run(x_bits, b, r0, n):
        import oracle as O
        F = {"e4m3": O.E4M3, "e5m2": O.E5M2, "e2m1": O.E2M1, "e2m3": O.E2M3, "e3m2": O.E3M2, "int8": O.INT8}[fmt]
        M = {"floor": O.FLOOR, "roundup": O.ROUNDUP}[mode]
        A = {"row": O.ROW, "col": O.COL, "both": O.BOTH}[axis]
        xs = x_bits[b, r0:r0 + n]
        if rounding == "rne" and block == "1x32":
            O.quantize(xs, dtype, F, M, A)
        else:
            R, C = x_bits.shape[1], x_bits.shape[2]
            O.quantize_ex(xs, dtype, F, M, A, rounding=rounding, seed=0x5EED, block=block,
                          first=(b * R + r0) * C)
    return run


def _cast_workload(gen, b, r, c, esize, fmt, mode, axis, desc, base, rounding="rne", block="1x32",
                   sources=None):
    """One quantize launch per step over one tensor; bytes = input + code and scale planes."""
    planes = 2 if axis == "both" else 1
    per_scale = 32 * 32 if block == "32x32" else 32
    n = b * r * c
    rd, wr = n * esize, planes * (n * CODE_BITS[fmt] // 8 + n // per_scale)

    def make(dev, i):
        import microscaling_block_quantized_amd as mx
        x = gen(dev, i).reshape(b, r, c)
        q = mx.BoundQuantize(x, fmt, mode, axis, _planes(dev, b, r, c, fmt, axis, block), rounding=rounding,
                             seed=0x5EED + i, block=block)
        return q, q
    cfg = {"workload": desc, "batch": b, "rows": r, "cols": c, "fmt": fmt, "scale_mode": mode, "axis": axis}
    if rounding != "rne" or block != "1x32":
        cfg.update(rounding=rounding, block=block)
    kname = _cast_kernel_name(esize == 2, fmt, mode, axis, rounding, block)
    return {"bytes": rd + wr, "make": make, "metric": f"GB/s (read+write), {desc}", "config": cfg,
            "dtype": "bf16" if esize == 2 else "f32", "base": base, "title": desc,
            "kernels": [(kname, kname, rd, wr)], "dominant": 0,
            "sources": sources or CAST_SOURCES,
            "cpu": {"gen": gen, "shape": (b, r, c), "slab": _mx_oracle_slab("bf16" if esize == 2 else "f32", fmt,
                                                                              mode, axis, rounding, block)}}


def _nvfp4_workload():
    """16384x4096 BF16 activations -> NVFP4, both copies, global scale computed
    in the same call (its amax pass reads the input a second time)."""
    b, r, c = 1, 16384, 4096
    n = b * r * c
    nbytes = 2 * n * 2 + 2 * (n // 2 + n // 16) + 4

    def make(dev, i):
        import torch
        import microscaling_block_quantized_amd as mx
        import mx_inputs as I
        x = I.activations(r, c, seed=1 + i, device=dev).view(b, r, c)

        def out():
            return {"global_scale": torch.empty((b,), dtype=torch.float32, device=dev),
                    "row_codes": torch.empty((b, r, c // 2), dtype=torch.uint8, device=dev),
                    "row_scales": torch.empty((b, r, c // 16), dtype=torch.uint8, device=dev),
                    "col_codes": torch.empty((b, c, r // 2), dtype=torch.uint8, device=dev),
                    "col_scales": torch.empty((b, c, r // 16), dtype=torch.uint8, device=dev)}
        step = mx.BoundQuantizeNvfp4(x, "both", out())
        given = out()
        given["global_scale"].copy_(mx.mx_quantize_nvfp4(x, "both")["global_scale"])
        cast_only = mx.BoundQuantizeNvfp4(x, "both", given, global_given=True)
        return step, cast_only
    desc = ("activations 16384x4096 bf16 -> NVFP4 (E2M1, 16-element UE4M3 blocks, FP32 global scale) row+col, "
            "global scale computed in the call")

    def prep(x_bits):
        import oracle as O
        return O.nvfp4_global_scale(O.widen(x_bits, "bf16"))         # the tensor-wide pass, once

    def slab(x_bits, bi, r0, rows, g):
        import oracle as O
        O.nvfp4_quantize(x_bits[bi, r0:r0 + rows], "bf16", O.BOTH, g)
    return {"bytes": nbytes, "make": make, "metric": f"GB/s (read+write), {desc}", "dtype": "bf16",
            "config": {"workload": desc, "batch": b, "rows": r, "cols": c, "fmt": "nvfp4", "axis": "both",
                       "input_reads": 2},
            "base": "nvfp4_cast_16384x4096", "title": "NVFP4 row+col cast with the global scale computed in the call, "
                                                     "16384x4096 BF16",
            "kernels": [("nv_cast_kernel<true, 3>", "nv_cast_kernel<bf16,row+col>", n * 2, 2 * (n // 2 + n // 16)),
                        ("nv_amax_kernel<true>", "nv_amax_kernel<bf16> (global amax, reads x)", n * 2, 0),
                        ("nv_zero_kernel", "nv_zero_kernel (clears g)", 0, 4)],
            "dominant": 0, "dominant_bytes": n * 2 + 2 * (n // 2 + n // 16),
            "sources": COMMON_SOURCES + [CSRC + "mx_nvfp4.hip", CSRC + "mx_cast_impl.h"],
            "cpu": {"gen": _gen("activations"), "shape": (b, r, c), "slab": slab, "prep": prep}}


def _requant_workload():
    """14336x4096 weights as MXFP4 (E2M1, floor, rows; made once, untimed) ->
    FP8 E4M3 with 128x128 block scales, both the row copy and the transposed
    copy, plus the per-block spread."""
    r, c = 14336, 4096
    n = r * c
    nblk = (r // 128) * (c // 128)
    rd, wr = n // 2 + n // 32, 2 * (n + 4 * nblk) + nblk

    def make(dev, i):
        import torch
        import microscaling_block_quantized_amd as mx
        import mx_inputs as I
        w = I.weights(r, c, seed=2 + 100 * i, device=dev)
        q = mx.mx_quantize(w, "e2m1", "floor", "row")
        del w
        out = {"e4m3": torch.empty((r, c), dtype=torch.uint8, device=dev),
               "block_scale": torch.empty((r // 128, c // 128), dtype=torch.float32, device=dev),
               "e4m3_t": torch.empty((c, r), dtype=torch.uint8, device=dev),
               "block_scale_t": torch.empty((c // 128, r // 128), dtype=torch.float32, device=dev),
               "spread": torch.empty((r // 128, c // 128), dtype=torch.uint8, device=dev)}
        s = mx.BoundRequant(q["row_codes"], q["row_scales"], (r, c), "both", out)
        return s, s
    desc = ("weights 14336x4096 as MXFP4 (E2M1 1x32, floor) -> FP8 E4M3 with 128x128 power-of-two block scales, "
            "row copy + transposed copy + scale-spread check")
    # 16 sets: 500 MB of MXFP4 inputs, so none is still in the 256 MB memory-side cache when its turn comes
    return {"bytes": rd + wr, "make": make, "metric": f"GB/s (read+write), {desc}", "sets": 16, "dtype": "u8",
            "config": {"workload": desc, "rows": r, "cols": c, "fmt": "e2m1->e4m3", "axis": "both"},
            "base": "fp4_in_fp8_requant_14336x4096", "title": "MXFP4 -> FP8 128x128 requantization, row + transposed "
                                                             "copy + spreads, 14336x4096",
            "kernels": [("requant_kernel<0, 0, true, true>", "requant_kernel<row+col>", rd, wr)], "dominant": 0,
            "sources": COMMON_SOURCES + [CSRC + "mx_requant.hip", CSRC + "mx_cast_impl.h"],
            "cpu": {"gen": lambda dev, i: _gen("weights")(dev, 0).view(1, r, c), "shape": (1, r, c),
                    "setup": _requant_setup, "slab": _requant_slab,
                    "note": "the MXFP4 plane made by the oracle beforehand, untimed"}}


def _requant_setup(x_bits):
    """The oracle's MXFP4 plane of the weights (E2M1 1x32, floor), codes and
    scales side by side: [1][R][C/2 + C/32] bytes."""
    import numpy as np
    import oracle as O
    q = O.quantize(x_bits, "bf16", O.E2M1, O.FLOOR, O.ROW)
    return np.concatenate([q["row_codes"], q["row_scales"]], axis=2)


def _requant_slab(src, b, r0, n):
    import oracle as O
    half = src.shape[2] * 16 // 17                               # C/2 of the C/2 + C/32 bytes
    O.requant_fp4_to_fp8(src[b:b + 1, r0:r0 + n, :half], src[b:b + 1, r0:r0 + n, half:])


def _qat_workload():
    """14336x4096 FP32 master weights -> MXFP4 (E2M1 1x32, floor) -> FP8 E4M3 with
    128x128 block scales, one pass: the MXFP4 plane, both FP8 copies and the
    spreads are written."""
    r, c = 14336, 4096
    n = r * c
    nblk = (r // 128) * (c // 128)
    rd, wr = 4 * n, (n // 2 + n // 32) + 2 * (n + 4 * nblk) + nblk

    def make(dev, i):
        import torch
        import microscaling_block_quantized_amd as mx
        import mx_inputs as I
        x = I.weights(r, c, seed=2 + 100 * i, device=dev).float()
        out = {"fp4_codes": torch.empty((r, c // 2), dtype=torch.uint8, device=dev),
               "fp4_scales": torch.empty((r, c // 32), dtype=torch.uint8, device=dev),
               "e4m3": torch.empty((r, c), dtype=torch.uint8, device=dev),
               "block_scale": torch.empty((r // 128, c // 128), dtype=torch.float32, device=dev),
               "e4m3_t": torch.empty((c, r), dtype=torch.uint8, device=dev),
               "block_scale_t": torch.empty((c // 128, r // 128), dtype=torch.float32, device=dev),
               "spread": torch.empty((r // 128, c // 128), dtype=torch.uint8, device=dev)}
        s = mx.BoundQuantizeFp4Fp8(x, "floor", "both", out)
        return s, s
    desc = ("FP32 master weights 14336x4096 -> MXFP4 (E2M1 1x32, floor) -> FP8 E4M3 with 128x128 power-of-two "
            "block scales in one pass: MXFP4 plane + row copy + transposed copy + spreads")
    return {"bytes": rd + wr, "make": make, "metric": f"GB/s (read+write), {desc}", "dtype": "f32",
            "config": {"workload": desc, "rows": r, "cols": c, "fmt": "f32->e2m1->e4m3", "axis": "both"},
            "base": "qat_fp32_fp4_fp8_14336x4096", "title": desc,
            "kernels": [("requant_kernel<2, 0, true, true>", "requant_kernel<fp32 master,row+col>", rd, wr)],
            "dominant": 0, "sources": COMMON_SOURCES + [CSRC + "mx_requant.hip", CSRC + "mx_cast_impl.h"],
            "cpu": {"gen": lambda dev, i: _gen("weights")(dev, 0).float().view(1, r, c), "shape": (1, r, c),
                    "slab": _qat_slab}}


def _qat_slab(x_bits, b, r0, n):
    import oracle as O
    q = O.quantize(x_bits[b, r0:r0 + n], "f32", O.E2M1, O.FLOOR, O.ROW)
    O.requant_fp4_to_fp8(q["row_codes"], q["row_scales"])


def _wide_range_pipeline():
    """64 x 4096x14336 BF16: fused E4M3 quantize, then both planes dequantized to BF16."""
    b, r, c = 64, 4096, 14336
    n = b * r * c
    q_rd, q_wr = n * 2, 2 * (n + n // 32)
    d_rd, d_wr = n + n // 32, n * 2
    nbytes = q_rd + q_wr + 2 * (d_rd + d_wr)

    def make(dev, i):
        import torch
        import microscaling_block_quantized_amd as mx
        import mx_inputs as I
        x = I.wide_range_batch(b, r, c, seed=4 + 100 * i, device=dev)
        planes = _planes(dev, b, r, c, "e4m3", "both")
        q = mx.BoundQuantize(x, "e4m3", "floor", "both", planes)
        yr = torch.empty((b, r, c), dtype=torch.bfloat16, device=dev)
        yc = torch.empty((b, c, r), dtype=torch.bfloat16, device=dev)
        dr = mx.BoundDequantize(planes["row_codes"], planes["row_scales"], "e4m3", (b, r, c), yr)
        dc = mx.BoundDequantize(planes["col_codes"], planes["col_scales"], "e4m3", (b, c, r), yc)

        def step():
            q()
            dr()
            dc()
        return step, q

    def slab(x_bits, bi, r0, rows):
        import oracle as O
        e = O.quantize(x_bits[bi, r0:r0 + rows], "bf16", O.E4M3, O.FLOOR, O.BOTH)
        O.dequantize(e["row_codes"], e["row_scales"], O.E4M3, "bf16")
        O.dequantize(e["col_codes"], e["col_scales"], O.E4M3, "bf16")
    return {"bytes": nbytes, "make": make, "sets": 1, "dtype": "bf16",
            "metric": "GB/s (read+write), 64x4096x14336 BF16 MXFP8 E4M3 row+col quantize + both dequantizes",
            "config": {"workload": "wide-range batch 64x4096x14336 bf16: fused E4M3 quantize (floor), then "
                                   "row and column planes dequantized to bf16",
                       "batch": b, "rows": r, "cols": c, "fmt": "e4m3", "scale_mode": "floor", "axis": "both"},
            "base": "wide_range_pipeline_64x4096x14336",
            "title": "wide-range batch 64x4096x14336 BF16: fused E4M3 quantize + both planes dequantized to BF16",
            "kernels": [("mx_cast_kernel<true, 0, 0, 3, 0, false>", "mx_cast_kernel<bf16,E4M3,floor,row+col>",
                         q_rd, q_wr),
                        ("mx_dequant_kernel<0, true, false>", "mx_dequant_kernel<E4M3,bf16> (per plane)", d_rd,
                         d_wr)],
            "dominant": 0, "sources": CAST_SOURCES + [CSRC + "mx_dequant.hip"],
            "cpu": {"gen": lambda dev, i: __import__("mx_inputs").wide_range_batch(4, r, c, seed=4, device=dev),
                    "shape": (4, r, c), "slab": slab, "extrapolate": b // 4}}


def _fp32_normal_round_trip():
    """256x1024 FP32 N(0,1): row-wise E4M3 quantize (floor) + dequantize to FP32."""
    r, c = 256, 1024
    n = r * c
    q_rd, q_wr = n * 4, n + n // 32
    d_rd, d_wr = n + n // 32, n * 4

    def make(dev, i):
        import torch
        import microscaling_block_quantized_amd as mx
        import mx_inputs as I
        x = I.fp32_normal(r, c, seed=i, device=dev)
        planes = _planes(dev, 1, r, c, "e4m3", "row")
        q = mx.BoundQuantize(x.view(1, r, c), "e4m3", "floor", "row", planes)
        y = torch.empty((1, r, c), dtype=torch.float32, device=dev)
        d = mx.BoundDequantize(planes["row_codes"], planes["row_scales"], "e4m3", (1, r, c), y)

        def step():
            q()
            d()
        return step, q

    def slab(x_bits, bi, r0, rows):
        import oracle as O
        e = O.quantize(x_bits[bi, r0:r0 + rows], "f32", O.E4M3, O.FLOOR, O.ROW)
        O.dequantize(e["row_codes"], e["row_scales"], O.E4M3, "f32")
    return {"bytes": q_rd + q_wr + d_rd + d_wr, "make": make, "dtype": "f32",
            "metric": "GB/s (read+write), 256x1024 FP32 MXFP8 E4M3 row quantize + dequantize",
            "config": {"workload": "fp32 N(0,1) 256x1024: row-wise E4M3 quantize (floor) + dequantize to fp32",
                       "rows": r, "cols": c, "fmt": "e4m3", "scale_mode": "floor", "axis": "row"},
            "base": "fp32_round_trip_256x1024",
            "title": "FP32 256x1024 row-wise E4M3 quantize + dequantize to FP32 (launch-bound)",
            "kernels": [("mx_cast_rows_kernel<false, 0, 0, 0>", "mx_cast_rows_kernel<f32,E4M3,floor>", q_rd, q_wr),
                        ("mx_dequant_kernel<0, false, false>", "mx_dequant_kernel<E4M3,f32>", d_rd, d_wr)],
            "dominant": 0, "sources": CAST_SOURCES + [CSRC + "mx_dequant.hip"],
            "cpu": {"gen": lambda dev, i: __import__("mx_inputs").fp32_normal(r, c, seed=0, device=dev).view(1, r, c),
                    "shape": (1, r, c), "slab": slab}}


WORKLOADS = {
    "activations": _cast_workload(_gen("activations"), 1, 16384, 4096, 2, "e4m3", "floor", "both",
                                  "activations 16384x4096 bf16 -> MXFP8 E4M3 row+col fused, floor scale rule",
                                  "fused_cast_e4m3_16384x4096"),
    "weights_floor": _cast_workload(_gen("weights"), 1, 14336, 4096, 2, "e2m1", "floor", "row",
                                    "weights 14336x4096 bf16 -> MXFP4 E2M1 row-wise, floor scale rule",
                                    "row_cast_e2m1_floor_14336x4096"),
    "weights_roundup": _cast_workload(_gen("weights"), 1, 14336, 4096, 2, "e2m1", "roundup", "row",
                                      "weights 14336x4096 bf16 -> MXFP4 E2M1 row-wise, round-up scale rule",
                                      "row_cast_e2m1_roundup_14336x4096"),
    "gradients": _cast_workload(_gen("gradients"), 1, 8192, 8192, 4, "e5m2", "roundup", "col",
                                "gradients 8192x8192 fp32 -> MXFP8 E5M2 column-wise, round-up scale rule",
                                "col_cast_e5m2_fp32_8192x8192"),
    "act_e2m3": _cast_workload(_gen("activations"), 1, 16384, 4096, 2, "e2m3", "floor", "both",
                               "activations 16384x4096 bf16 -> MXFP6 E2M3 row+col fused, floor scale rule",
                               "fused_cast_e2m3_16384x4096"),
    "act_e3m2": _cast_workload(_gen("activations"), 1, 16384, 4096, 2, "e3m2", "floor", "both",
                               "activations 16384x4096 bf16 -> MXFP6 E3M2 row+col fused, floor scale rule",
                               "fused_cast_e3m2_16384x4096"),
    "act_int8": _cast_workload(_gen("activations"), 1, 16384, 4096, 2, "int8", "floor", "both",
                               "activations 16384x4096 bf16 -> MXINT8 row+col fused, floor scale rule",
                               "fused_cast_int8_16384x4096"),
    "grad_sr_e2m1": _cast_workload(_gen("gradients"), 1, 8192, 8192, 4, "e2m1", "roundup", "col",
                                   "gradients 8192x8192 fp32 -> MXFP4 E2M1 column-wise, stochastic rounding, "
                                   "round-up scale rule", "col_cast_sr_e2m1_fp32_8192x8192", rounding="sr",
                                   sources=CAST_SOURCES + [CSRC + "mx_cast_sr.hip"]),
    "weights_2d_e2m1": _cast_workload(_gen("weights"), 1, 14336, 4096, 2, "e2m1", "floor", "both",
                                      "weights 14336x4096 bf16 -> MXFP4 E2M1 32x32 blocks, row+col fused, "
                                      "floor scale rule", "cast_2d_e2m1_14336x4096", block="32x32",
                                      sources=CAST_SOURCES + [CSRC + "mx_cast_2d.hip"]),
    "act_nvfp4": _nvfp4_workload(),
    "weights_fp4_in_fp8": _requant_workload(),
    "qat_fp4_fp8": _qat_workload(),
    "wide_range": _wide_range_pipeline(),
    "fp32_normal": _fp32_normal_round_trip(),
}
METRIC = "GB/s (read+write) and % of HBM peak, MXFP8 row+col cast 16384×4096"
# workloads whose main kernel is bound by VALU work and its latency, not HBM
ALU_BOUND = ("grad_sr_e2m1", "act_nvfp4")


# ---------------------------------------------------------------------------
# profile summaries (rocprofv3 output -> profiles/*.md, *.txt)
# ---------------------------------------------------------------------------

def kernel_hash(workload: str) -> str:
    h = hashlib.sha256()
    for p in WORKLOADS[workload]["sources"]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counters_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", WORKLOADS[workload]["base"] + "_counters.txt")


def read_counters(workload: str):
    """HBM bytes per launch of the workload's dominant kernel from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source."""
    path = counters_path(workload)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(("#", "|")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_hash") != kernel_hash(workload):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def summarize_trace(stats_csv: str, command: str, workload: str) -> str:
    """Text summary of a rocprofv3 --kernel-trace --stats run (kernel_stats.csv)."""
    wl = WORKLOADS[workload]
    copy_each_way = copy_bytes(wl["bytes"])
    out = [f"# rocprofv3 kernel trace: {wl['title']}", "",
           f"command: {command}", "", "| kernel | calls | average us | min us | max us | algorithmic GB/s |",
           "|---|---|---|---|---|---|"]
    for r in _csv_rows(stats_csv):
        name = r["Name"]
        hit = [(short, rd + wr) for sub_, short, rd, wr in wl["kernels"] if sub_ in name]
        if hit:
            short, nbytes = hit[0]
        elif COPY_KERNEL in name:
            short, nbytes = "torch device copy (" + COPY_KERNEL + ")", 2 * copy_each_way
        elif LIB_COPY_KERNEL in name:
            short, nbytes = "libmx non-temporal copy (" + LIB_COPY_KERNEL + ", the ceiling)", 2 * copy_each_way
        else:
            continue
        avg = float(r["AverageNs"]) / 1e3
        gbs = f"{nbytes / (avg * 1e-6) / 1e9:.1f}" if nbytes else "-"
        out.append(f"| {short} | {r['Calls']} | {avg:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                   f"{float(r['MaxNs']) / 1e3:.2f} | {gbs} |")
    return "\n".join(out) + "\n"


CALIBRATION_COPIES = 30      # the timed torch copies of known size at the end of every bench run


def _counter_means(path, counter, keys):
    """Mean counter value per kernel. For torch's copy kernel only the last
    CALIBRATION_COPIES dispatches count: those are the bench's own copies of a
    known size (input set-up makes other, smaller copies earlier in the run)."""
    acc = {}
    rows = sorted((r for r in _csv_rows(path) if r["Counter_Name"] == counter), key=lambda r: int(r["Dispatch_Id"]))
    for r in rows:
        for sub_, key in keys:
            if sub_ in r["Kernel_Name"]:
                acc.setdefault(key, []).append(float(r["Counter_Value"]))
                break
    if "copy" in acc:
        acc["copy"] = acc["copy"][-CALIBRATION_COPIES:]
    return {k: sum(v) / len(v) for k, v in acc.items()}


def summarize_counters(fetch_csv: str, write_csv: str, command: str, workload: str) -> str:
    """Per-kernel HBM bytes per launch from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for torch's copy kernel
    moving a known number of bytes in the same run."""
    wl = WORKLOADS[workload]
    keys = [(k[0], k[1]) for k in wl["kernels"]] + [(COPY_KERNEL, "copy")]
    copy_each_way = copy_bytes(wl["bytes"])
    f = _counter_means(fetch_csv, "FETCH_SIZE", keys)
    w = _counter_means(write_csv, "WRITE_SIZE", keys)
    f_cal = copy_each_way / (f["copy"] * 1024.0)
    w_cal = copy_each_way / (w["copy"] * 1024.0)
    lines = [f"# rocprofv3 HBM counters: {wl['title']}", "",
             f"command (FETCH_SIZE): {command.format(counter='FETCH_SIZE')}",
             f"command (WRITE_SIZE): {command.format(counter='WRITE_SIZE')}", "",
             f"calibration: torch copy kernel {COPY_KERNEL} moving {copy_each_way} B each way reads "
             f"FETCH_SIZE {f['copy']:.1f} KiB (factor {f_cal:.4f}) and WRITE_SIZE {w['copy']:.1f} KiB "
             f"(factor {w_cal:.4f})", "",
             "| kernel | fetched B (calibrated) | algorithmic read | ratio | written B (calibrated) | "
             "algorithmic write | ratio |", "|---|---|---|---|---|---|---|"]
    dom = None
    for i, (_, short, rd, wr) in enumerate(wl["kernels"]):
        if short not in f or short not in w:
            continue
        fb = f[short] * 1024.0 * f_cal
        wb = w[short] * 1024.0 * w_cal
        lines.append(f"| {short} | {fb:.0f} | {rd} | {(fb / rd) if rd else float('nan'):.4f} | {wb:.0f} | {wr} | "
                     f"{(wb / wr) if wr else float('nan'):.4f} |")
        if i == wl["dominant"]:
            dom = (short, fb + wb)
    lines += ["", f"dominant_kernel: {dom[0]}", f"hbm_bytes_per_launch: {dom[1]:.0f}",
              f"kernel_source_hash: {kernel_hash(workload)}"]
    return "\n".join(lines) + "\n"


# main kernel and element count of the workloads with SQ (instruction) counter summaries
SQ_ELEMENTS = {"activations": 16384 * 4096, "act_e2m3": 16384 * 4096, "act_nvfp4": 16384 * 4096,
               "grad_sr_e2m1": 8192 * 8192, "weights_fp4_in_fp8": 14336 * 4096, "qat_fp4_fp8": 14336 * 4096}
SQ_PROFILE = os.path.join(ROOT, "profiles", "valu_lds_counters.md")
SQ_COUNTERS = ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT",
               "SQ_INSTS_VMEM_RD", "SQ_INSTS_VMEM_WR")


def valu_ops_per_element(workload: str):
    """VALU lane-ops per element of the workload's dominant kernel, from the
    committed instruction-counter summary, or None."""
    if not os.path.exists(SQ_PROFILE):
        return None
    with open(SQ_PROFILE) as f:
        for line in f:
            cells = [c.strip() for c in line.strip().strip("|").split("|")]
            if len(cells) >= 5 and cells[0] == workload:
                try:
                    return float(cells[4])
                except ValueError:
                    return None
    return None


def _counter_means_all(path, kernel_sub):
    acc = {}
    for r in _csv_rows(path):
        if kernel_sub in r["Kernel_Name"]:
            acc.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def summarize_sq(command: str, csvs: list) -> str:
    """Instruction counters per dispatch of each workload's dominant kernel, from
    rocprofv3 --pmc runs of the SQ_COUNTERS (one CSV per workload, named
    .../sq_<workload>/...). VALU lane-ops per element = SQ_INSTS_VALU * 64 / elements."""
    out = ["# rocprofv3 instruction counters: VALU work per element and LDS bank conflicts", "",
           f"command (per workload W): {command}", "",
           "| workload | kernel | waves | VALU instr per wave | VALU lane-ops per element | SALU per wave | "
           "LDS instr per wave | LDS bank-conflict cycles per LDS instr |", "|---|---|---|---|---|---|---|---|"]
    for path in csvs:
        w = next(k for k in SQ_ELEMENTS if f"sq_{k}/" in path or f"sq_{k}\\" in path)
        wl = WORKLOADS[w]
        sub_ = wl["kernels"][wl["dominant"]][0]
        m = _counter_means_all(path, sub_)
        waves = m["SQ_WAVES"]
        out.append(f"| {w} | {sub_} | {waves:.0f} | {m['SQ_INSTS_VALU'] / waves:.1f} | "
                   f"{m['SQ_INSTS_VALU'] * 64 / SQ_ELEMENTS[w]:.2f} | {m['SQ_INSTS_SALU'] / waves:.1f} | "
                   f"{m['SQ_INSTS_LDS'] / waves:.1f} | {m['SQ_LDS_BANK_CONFLICT'] / max(m['SQ_INSTS_LDS'], 1):.2f} |")
    return "\n".join(out) + "\n"


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on the host cores
# ---------------------------------------------------------------------------

def _cpu_model() -> str:
    """The host CPU as lscpu describes it: the model name (which a virtual machine
    may shorten, e.g. to "AMD EPYC") with the family / model / stepping numbers
    and the topology that identify it."""
    info = {}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if ":" in line:
                k, v = line.split(":", 1)
                info[k.strip()] = v.strip()
    except (OSError, subprocess.SubprocessError):
        pass
    name = info.get("Model name")
    if not name:
        try:
            with open("/proc/cpuinfo") as f:
                for line in f:
                    if line.startswith("model name"):
                        name = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
    fields = [("family", "CPU family"), ("model", "Model"), ("stepping", "Stepping"), ("sockets", "Socket(s)"),
              ("cores/socket", "Core(s) per socket"), ("threads/core", "Thread(s) per core"),
              ("max MHz", "CPU max MHz")]
    extra = ", ".join(f"{label} {info[key]}" for label, key in fields if info.get(key))
    return f"{name or 'unknown'} ({extra})" if extra else (name or "unknown")


_CPU_JOB = None


def _cpu_task(task):
    b, r0, n = task
    if _CPU_JOB["state"] is None:
        _CPU_JOB["slab"](_CPU_JOB["x"], b, r0, n)
    else:
        _CPU_JOB["slab"](_CPU_JOB["x"], b, r0, n, _CPU_JOB["state"])
    return n


def cpu_baselines(workload: str, dev, procs: int, single_budget_s: float = 10.0):
    """The oracle on the same workload: over every 512-row slab in `procs` forked
    processes (the workers touch only host memory), and on one core over a
    bounded sample of slabs. GB/s on the workload's algorithmic-byte basis."""
    import multiprocessing as mp
    import mx_inputs as I
    global _CPU_JOB
    wl = WORKLOADS[workload]
    cpu = wl["cpu"]
    if cpu is None:
        return None, None
    B, R, C = cpu["shape"]
    x = I.to_bits(cpu["gen"](dev, 0)).reshape(B, R, C)
    if "setup" in cpu:                     # the workload's own input, made by the oracle (untimed)
        x = cpu["setup"](x)
    note = f", {cpu['note']}" if "note" in cpu else ""
    ext = cpu.get("extrapolate", 1)
    per_row = wl["bytes"] / (B * ext * R)
    slab = 512
    tasks = [(b, r0, min(slab, R - r0)) for b in range(B) for r0 in range(0, R, slab)]
    t_prep, state = 0.0, None
    if "prep" in cpu:                      # a pass over the whole input that every slab needs (one process)
        t0 = time.perf_counter()
        state = cpu["prep"](x)
        t_prep = time.perf_counter() - t0
    _CPU_JOB = {"x": x, "slab": cpu["slab"], "state": state}
    try:
        done, t_used = 0, 0.0
        for t in tasks:
            if t_used >= single_budget_s:
                break
            t0 = time.perf_counter()
            _cpu_task(t)
            t_used += time.perf_counter() - t0
            done += t[2]
        frac = done / (B * R)
        t_single = t_used + t_prep * frac
        single = {"value": round(per_row * done / t_single / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                  "sample": f"{done} rows of {B * R} ({'tensor batch of ' + str(B) if B > 1 else 'one tensor'}) in "
                            f"512-row slabs, NumPy float64 oracle, one process, {t_single:.1f} s{note}"}
        par = None
        if procs > 1:
            with mp.get_context("fork").Pool(procs) as pool:
                pool.map(_cpu_task, tasks[:procs], chunksize=1)            # start the workers
                t0 = time.perf_counter()
                pool.map(_cpu_task, tasks, chunksize=1)
                t = time.perf_counter() - t0 + t_prep
            try:
                affinity = len(os.sched_getaffinity(0))
            except AttributeError:
                affinity = None
            span = (f"all {B * R} rows" if ext == 1 else
                    f"{B} of {B * ext} tensors, timed and scaled x{ext} (extrapolated)")
            par = {"value": round(wl["bytes"] / (t * ext) / 1e9, 4), "unit": "GB/s", "cores": procs, "kind": "oracle",
                   "sample": f"{span} in 512-row slabs over {procs} forked processes, NumPy float64 oracle, "
                             f"{t:.2f} s{note}",
                   "extrapolated": ext != 1, "host_logical_cpus": os.cpu_count(), "affinity_cpus": affinity,
                   "cpu_model": _cpu_model(),
                   "procs_note": f"pool of min({CPU_PROCS}, host CPUs): {CPU_PROCS} processes are this GPU's share "
                                 "of the host"}
        return par, single
    finally:
        _CPU_JOB = None


# ---------------------------------------------------------------------------
# main
# ---------------------------------------------------------------------------

def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=0,
                    help="rotating input/output buffer sets (default per workload: 8; 16 for the "
                         "requantization; 1 for the 30 GB wide-range batch)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-procs", type=int, default=CPU_PROCS,
                    help="worker processes of the oracle baseline (the box's CPU share for one GPU), capped at the "
                         "host's CPUs; 1 times one process only")
    ap.add_argument("--workload", default="activations", choices=sorted(WORKLOADS),
                    help="activations (default) is the fused row+col MXFP8 cast the metric is quoted on; "
                         "the others time the remaining workloads the same way")
    ap.add_argument("--summarize-trace", metavar="KERNEL_STATS_CSV",
                    help="print a summary of a rocprofv3 --kernel-trace --stats run and exit")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the calibrated HBM-traffic summary of two rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-sq", nargs="+", metavar="COUNTER_CSV",
                    help="print the VALU / LDS instruction-counter summary of rocprofv3 --pmc runs and exit")
    ap.add_argument("--command", default="", help="command line recorded in a summary")
    ap.add_argument("--trace-workload", default="activations", choices=sorted(WORKLOADS),
                    help="which workload's kernels --summarize-trace / --summarize-counters report")
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.command, args.trace_workload), end="")
        return 0
    if args.summarize_sq:
        print(summarize_sq(args.command, args.summarize_sq), end="")
        return 0
    if args.summarize_counters:
        print(summarize_counters(*args.summarize_counters, args.command, args.trace_workload), end="")
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the MX cast needs no "
              "cross-GPU exchange, so run it once per GPU.", file=sys.stderr)
        return 2

    import torch

    import microscaling_block_quantized_amd as mx

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = WORKLOADS[args.workload]
    if args.sets <= 0:
        args.sets = wl.get("sets", 8)
    made = [wl["make"](dev, i) for i in range(args.sets)]
    steps_fns = [m[0] for m in made]
    dominant_fns = [m[1] for m in made]
    torch.cuda.synchronize()

    # device warm-up to steady clocks (untimed, at least 150 ms of the same step)
    t_end = time.perf_counter() + 0.15
    i = 0
    while time.perf_counter() < t_end or i < args.sets:
        steps_fns[i % args.sets]()
        if i % 16 == 15:
            torch.cuda.synchronize()
        i += 1
    torch.cuda.synchronize()
    for i in range(args.warmup):
        steps_fns[i % args.sets]()
    torch.cuda.synchronize()

    # the timed region: K steps between two events on the launch stream
    stream = torch.cuda.current_stream(dev)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        steps_fns[i % args.sets]()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    alg_bytes = wl["bytes"]

    # the dominant kernel alone, where a step launches more than one kernel
    dom_bytes = wl.get("dominant_bytes")
    if dom_bytes is None:
        _, _, rd, wr = wl["kernels"][wl["dominant"]]
        dom_bytes = rd + wr
    if dominant_fns[0] is steps_fns[0]:
        dom_us = ms * 1e3
    else:
        k = max(args.steps // 4, 8)
        for i in range(4):
            dominant_fns[i % args.sets]()
        d0 = torch.cuda.Event(enable_timing=True)
        d1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        d0.record(stream)
        for i in range(k):
            dominant_fns[i % args.sets]()
        d1.record(stream)
        torch.cuda.synchronize()
        dom_us = d0.elapsed_time(d1) / k * 1e3

    # spread of single steps (outside the timed region): 64 steps, each between its own events
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(64)]
    for i, (e0, e1) in enumerate(evs):
        e0.record(stream)
        steps_fns[i % args.sets]()
        e1.record(stream)
    torch.cuda.synchronize()
    one = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)
    per_launch = {"p10": round(one[6], 2), "p50": round(one[32], 2), "p90": round(one[57], 2), "unit": "us",
                  "samples": len(one)}
    del steps_fns, dominant_fns, made
    torch.cuda.empty_cache()

    # Measured ceilings: the library's plain non-temporal 16-byte copy (the same
    # kind of read and write traffic with no arithmetic), and torch's device copy,
    # whose kernel the HBM-counter summaries use for calibration.
    copy_half = copy_bytes(alg_bytes)
    src = torch.empty(copy_half, dtype=torch.uint8, device=dev)
    dsts = [torch.empty_like(src) for _ in range(3)]
    for d in dsts:
        d.copy_(src)
        mx.mx_copy_nt(src, d)
    torch.cuda.synchronize()

    def time_copies(fn):
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for i in range(30):
            fn(dsts[i % 3])
        c1.record(stream)
        torch.cuda.synchronize()
        return 2 * copy_half / (c0.elapsed_time(c1) / 30 * 1e-3) / 1e9

    torch_copy_gbs = time_copies(lambda d: d.copy_(src))
    copy_gbs = time_copies(lambda d: mx.mx_copy_nt(src, d))
    del src, dsts

    gbs = alg_bytes / (ms * 1e-3) / 1e9
    dom_gbs = dom_bytes / (dom_us * 1e-6) / 1e9
    dom_name = wl["kernels"][wl["dominant"]][1]
    line = {
        "metric": METRIC if args.workload == "activations" else wl["metric"],
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.get("dtype", "bf16"),
        "data": "synthetic",
        "config": dict(wl["config"], buffer_sets=args.sets, alg_bytes_per_step=alg_bytes),
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "per_launch_us": per_launch,
        "roofline": {"bound": "hbm", "achieved": round(dom_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dom_gbs / HBM_PEAK_GBS, 4), "traffic": read_counters(args.workload),
                     "kernel": dom_name, "alg_bytes_per_launch": dom_bytes, "avg_launch_us": round(dom_us, 3)},
        "copy_ceiling": {"value": round(copy_gbs, 2), "unit": "GB/s",
                         "what": f"libmx non-temporal 16-byte copy (mx_copy_nt), {copy_half} B each way, "
                                 "3 rotating destinations",
                         "frac_of_ceiling": round(gbs / copy_gbs, 4),
                         "torch_device_copy": round(torch_copy_gbs, 2)},
    }
    ops = valu_ops_per_element(args.workload) if args.workload in ALU_BOUND else None
    if ops is not None:
        # VALU-bound: the roofline is the VALU issue rate; the HBM view stays beside it
        elems = SQ_ELEMENTS[args.workload]
        tops = ops * elems / (dom_us * 1e-6) / 1e12
        line["hbm_roofline"] = line["roofline"]
        line["roofline"] = {"bound": "alu", "achieved": round(tops, 3), "peak": round(VALU_PEAK_T_LANE_OPS, 2),
                            "unit": "T VALU lane-ops/s", "frac": round(tops / VALU_PEAK_T_LANE_OPS, 4),
                            "traffic": None, "valu_lane_ops_per_element": ops, "kernel": dom_name,
                            "avg_launch_us": round(dom_us, 3),
                            "source": "profiles/valu_lds_counters.md (SQ_INSTS_VALU x 64 / elements)"}
    if not args.no_cpu_baseline:
        procs = max(1, min(args.cpu_procs, os.cpu_count() or 1))
        par, single = cpu_baselines(args.workload, dev, procs)
        if par is not None or single is not None:
            line["cpu_baseline"] = par if par is not None else single
            line["cpu_baseline_single"] = single
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
