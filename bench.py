"""Throughput of the fused row+column MXFP8 cast on one MI355X.

Workload: a 16384x4096 BF16 activation tensor (N(0,1) with 4 outlier columns
x100, seeded, synthetic), quantized to MXFP8 E4M3 with the OCP floor scale
rule, row-wise and column-wise (transposed) copies emitted by one kernel. One
step = one such cast over one tensor, inputs already resident in HBM. Eight
input/output buffer sets rotate (2.2 GB), so nothing a step reads or writes is
still in the 256 MB last-level cache when that set comes round again. Before
the W warm-up steps the GPU runs the same step for at least 150 ms, untimed,
so the timed steps run at steady clocks.

Prints one JSON line. `value` is GB/s of algorithmic traffic (each input byte
read once, each code and scale byte written once: 272,629,760 B per step).
`roofline` compares that rate with MI355X's 8 TB/s HBM peak; `traffic`
carries the HBM bytes per launch that rocprofv3 counters measured for the same
kernel source (profiles/), or null if the kernel changed since. `cpu_baseline`
times the CPU oracle, single-threaded, on a bounded slab of the same tensor;
`cpu_baseline_parallel` times it over the whole tensor in up to 16 forked
processes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

ROWS, COLS = 16384, 4096
ALG_BYTES = ROWS * COLS * 2 + 2 * (ROWS * COLS + ROWS * COLS // 32)   # 272,629,760
HBM_PEAK_GBS = 8000.0
METRIC = "GB/s (read+write) and % of HBM peak, MXFP8 row+col cast 16384×4096"
COUNTERS = os.path.join(ROOT, "profiles", "fused_cast_e4m3_16384x4096_counters.txt")
KERNEL_SOURCES = ["microscaling_block_quantized_amd/csrc/mx_cast.hip",
                  "microscaling_block_quantized_amd/csrc/mx_api.cpp",
                  "microscaling_block_quantized_amd/csrc/mx_kernels.h",
                  "microscaling_block_quantized_amd/csrc/mx_cast_impl.h",
                  "microscaling_block_quantized_amd/csrc/mx_sr.h",
                  "microscaling_block_quantized_amd/csrc/mx_device.h"]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_counters():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source."""
    if not os.path.exists(COUNTERS):
        return None
    kv = {}
    with open(COUNTERS) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_hash") != kernel_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


COPY_KERNEL = "__amd_rocclr_copyBuffer"
LIB_COPY_KERNEL = "copy_nt_kernel"
def copy_bytes(alg_bytes: int) -> int:
    """Bytes each way of the ceiling copy: the workload's read+write byte count,
    but at least 256 MiB each way so four buffers exceed the 256 MB cache."""
    return min(max(alg_bytes // 2, 1 << 28), 1 << 31)


COPY_BYTES = copy_bytes(ALG_BYTES)   # each ceiling copy of the fused workload reads and writes this much
CAST_KERNEL = "mx_cast_kernel<true, 0, 0, 3, 0, false>"


def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


_NV_N = ROWS * COLS
_RQ_N = 14336 * 4096
# per workload: (kernel-name substring, short name, algorithmic bytes per launch)
TRACE_KERNELS = {
    "activations": ("fused MXFP8 E4M3 row+col cast, 16384x4096 BF16",
                    [(CAST_KERNEL, "mx_cast_kernel<bf16,E4M3,floor,row+col>", ALG_BYTES)]),
    "act_nvfp4": ("NVFP4 row+col cast with the global scale computed in the call, 16384x4096 BF16",
                  [("nv_amax_kernel<true>", "nv_amax_kernel<bf16> (global amax, reads x)", _NV_N * 2),
                   ("nv_cast_kernel<true, 3>", "nv_cast_kernel<bf16,row+col>",
                    _NV_N * 2 + 2 * (_NV_N // 2 + _NV_N // 16)),
                   ("nv_zero_kernel", "nv_zero_kernel (clears g)", 4)]),
    "act_e2m3": ("fused MXFP6 E2M3 row+col cast, 16384x4096 BF16",
                 [("mx_cast_kernel<true, 3, 0, 3, 0, false>", "mx_cast_kernel<bf16,E2M3,floor,row+col>",
                   _NV_N * 2 + 2 * (_NV_N * 3 // 4 + _NV_N // 32))]),
    "act_int8": ("fused MXINT8 row+col cast, 16384x4096 BF16",
                 [("mx_cast_kernel<true, 5, 0, 3, 0, false>", "mx_cast_kernel<bf16,INT8,floor,row+col>",
                   _NV_N * 2 + 2 * (_NV_N + _NV_N // 32))]),
    "weights_2d_e2m1": ("MXFP4 E2M1 32x32-block row+col cast, 14336x4096 BF16",
                        [("mx_cast_kernel<true, 2, 0, 3, 0, true>", "mx_cast_kernel<bf16,E2M1,floor,row+col,32x32>",
                          _RQ_N * 2 + 2 * (_RQ_N // 2 + _RQ_N // 1024))]),
    "weights_fp4_in_fp8": ("MXFP4 -> FP8 128x128 requantization, row + transposed copy + spreads, 14336x4096",
                           [("requant_kernel<0, 0, true, true>", "requant_kernel<row+col>",
                             _RQ_N // 2 + _RQ_N // 32 + 2 * (_RQ_N + 4 * (_RQ_N // 16384)) + _RQ_N // 16384)]),
}


def summarize_trace(stats_csv: str, command: str, workload: str = "activations") -> str:
    """Text summary of a rocprofv3 --kernel-trace --stats run (kernel_stats.csv)."""
    title, kernels = TRACE_KERNELS[workload]
    copy_each_way = copy_bytes(WORKLOADS[workload]["bytes"])
    out = [f"# rocprofv3 kernel trace: {title}", "",
           f"command: {command}", "", "| kernel | calls | average us | min us | max us | algorithmic GB/s |",
           "|---|---|---|---|---|---|"]
    for r in _csv_rows(stats_csv):
        name = r["Name"]
        hit = [(short, nb) for sub_, short, nb in kernels if sub_ in name]
        if hit:
            short, nbytes = hit[0]
        elif COPY_KERNEL in name:
            short, nbytes = "torch device copy (" + COPY_KERNEL + ")", 2 * copy_each_way
        elif LIB_COPY_KERNEL in name:
            short, nbytes = "libmx non-temporal copy (" + LIB_COPY_KERNEL + ", the ceiling)", 2 * copy_each_way
        else:
            continue
        avg = float(r["AverageNs"]) / 1e3
        out.append(f"| {short} | {r['Calls']} | {avg:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                   f"{float(r['MaxNs']) / 1e3:.2f} | {nbytes / (avg * 1e-6) / 1e9:.1f} |")
    return "\n".join(out) + "\n"


# per workload, for the counter summaries: (kernel-name substring, short name,
# algorithmic bytes read, algorithmic bytes written) per launch
COUNTER_KERNELS = {
    "act_e2m3": [("mx_cast_kernel<true, 3, 0, 3, 0, false>", "mx_cast_kernel<bf16,E2M3,floor,row+col>", _NV_N * 2,
                  2 * (_NV_N * 3 // 4 + _NV_N // 32))],
    "act_int8": [("mx_cast_kernel<true, 5, 0, 3, 0, false>", "mx_cast_kernel<bf16,INT8,floor,row+col>", _NV_N * 2,
                  2 * (_NV_N + _NV_N // 32))],
    "weights_2d_e2m1": [("mx_cast_kernel<true, 2, 0, 3, 0, true>", "mx_cast_kernel<bf16,E2M1,floor,row+col,32x32>",
                         _RQ_N * 2, 2 * (_RQ_N // 2 + _RQ_N // 1024))],
    "act_nvfp4": [("nv_amax_kernel<true>", "nv_amax_kernel<bf16>", _NV_N * 2, 0),
                  ("nv_cast_kernel<true, 3>", "nv_cast_kernel<bf16,row+col>", _NV_N * 2, 2 * (_NV_N // 2 + _NV_N // 16))],
    "weights_fp4_in_fp8": [("requant_kernel<0, 0, true, true>", "requant_kernel<row+col>", _RQ_N // 2 + _RQ_N // 32,
                            2 * (_RQ_N + 4 * (_RQ_N // 16384)) + _RQ_N // 16384)],
}


def _counter_means(path, counter, keys):
    acc = {}
    for r in _csv_rows(path):
        if r["Counter_Name"] != counter:
            continue
        for sub_, key in keys:
            if sub_ in r["Kernel_Name"]:
                acc.setdefault(key, []).append(float(r["Counter_Value"]))
                break
    return {k: sum(v) / len(v) for k, v in acc.items()}


def summarize_counters_of(fetch_csv: str, write_csv: str, command: str, workload: str) -> str:
    """Per-kernel calibrated HBM bytes for one of the other workloads (see summarize_counters)."""
    kernels = COUNTER_KERNELS[workload]
    keys = [(k[0], k[1]) for k in kernels] + [(COPY_KERNEL, "copy")]
    copy_each_way = copy_bytes(WORKLOADS[workload]["bytes"])
    f = _counter_means(fetch_csv, "FETCH_SIZE", keys)
    w = _counter_means(write_csv, "WRITE_SIZE", keys)
    f_cal = copy_each_way / (f["copy"] * 1024.0)
    w_cal = copy_each_way / (w["copy"] * 1024.0)
    lines = [f"# rocprofv3 HBM counters: {TRACE_KERNELS[workload][0]}", "",
             f"command (FETCH_SIZE): {command.format(counter='FETCH_SIZE')}",
             f"command (WRITE_SIZE): {command.format(counter='WRITE_SIZE')}", "",
             f"calibration: torch copy kernel {COPY_KERNEL} moving {copy_each_way} B each way reads "
             f"FETCH_SIZE {f['copy']:.1f} KiB (factor {f_cal:.4f}) and WRITE_SIZE {w['copy']:.1f} KiB "
             f"(factor {w_cal:.4f})", "",
             "| kernel | fetched B (calibrated) | algorithmic read | ratio | written B (calibrated) | "
             "algorithmic write | ratio |", "|---|---|---|---|---|---|---|"]
    for _, short, rd, wr in kernels:
        fb = f[short] * 1024.0 * f_cal
        wb = w[short] * 1024.0 * w_cal
        lines.append(f"| {short} | {fb:.0f} | {rd} | {fb / rd:.4f} | {wb:.0f} | {wr} | "
                     f"{(wb / wr) if wr else float('nan'):.4f} |")
    return "\n".join(lines) + "\n"


# main kernel and element count of the workloads with SQ (instruction) counter summaries
SQ_KERNELS = {
    "activations": (CAST_KERNEL, ROWS * COLS),
    "act_e2m3": ("mx_cast_kernel<true, 3, 0, 3, 0, false>", ROWS * COLS),
    "grad_sr_e2m1": ("mx_cast_kernel<false, 2, 1, 2, 1, false>", 8192 * 8192),
}
# VALU issue peak of MI355X, non-packed: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
VALU_PEAK_T_LANE_OPS = 256 * 4 * 16 * 2.4e9 / 1e12          # 39.32 T lane-ops/s
# workloads whose main kernel is bound by VALU work and its latency, not HBM
ALU_BOUND = ("grad_sr_e2m1",)
SQ_PROFILE = os.path.join(ROOT, "profiles", "valu_lds_counters.md")


def valu_ops_per_element(workload: str):
    """VALU lane-ops per element of the workload's main kernel, from the committed
    instruction-counter summary, or None."""
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


SQ_COUNTERS = ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT",
               "SQ_INSTS_VMEM_RD", "SQ_INSTS_VMEM_WR")


def summarize_sq(command: str, csvs: list) -> str:
    """Instruction counters per dispatch of each workload's main kernel, from
    rocprofv3 --pmc runs of the SQ_COUNTERS (one CSV per workload, named
    .../sq_<workload>/...). VALU lane-ops per element = SQ_INSTS_VALU * 64 / elements."""
    out = ["# rocprofv3 instruction counters: VALU work per element and LDS bank conflicts", "",
           f"command (per workload W): {command}", "",
           "| workload | kernel | waves | VALU instr per wave | VALU lane-ops per element | SALU per wave | "
           "LDS instr per wave | LDS bank-conflict cycles per LDS instr |", "|---|---|---|---|---|---|---|---|"]
    for path in csvs:
        w = next(k for k in SQ_KERNELS if f"sq_{k}" in path)
        sub_, n = SQ_KERNELS[w]
        m = _counter_means_all(path, sub_)
        waves = m["SQ_WAVES"]
        out.append(f"| {w} | {sub_} | {waves:.0f} | {m['SQ_INSTS_VALU'] / waves:.1f} | "
                   f"{m['SQ_INSTS_VALU'] * 64 / n:.2f} | {m['SQ_INSTS_SALU'] / waves:.1f} | "
                   f"{m['SQ_INSTS_LDS'] / waves:.1f} | {m['SQ_LDS_BANK_CONFLICT'] / max(m['SQ_INSTS_LDS'], 1):.2f} |")
    return "\n".join(out) + "\n"


def _counter_means_all(path, kernel_sub):
    acc = {}
    for r in _csv_rows(path):
        if kernel_sub in r["Kernel_Name"]:
            acc.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def summarize_counters(fetch_csv: str, write_csv: str, command: str) -> str:
    """HBM bytes per launch of the cast from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for torch's copy kernel
    moving a known number of bytes in the same run."""
    def per_kernel(path, counter):
        return _counter_means(path, counter, [(CAST_KERNEL, "cast"), (COPY_KERNEL, "copy")])
    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    f_cal = COPY_BYTES / (f["copy"] * 1024.0)
    w_cal = COPY_BYTES / (w["copy"] * 1024.0)
    fetch_b = f["cast"] * 1024.0 * f_cal
    write_b = w["cast"] * 1024.0 * w_cal
    alg_read = ROWS * COLS * 2
    alg_write = ALG_BYTES - alg_read
    lines = [
        "# rocprofv3 HBM counters: fused MXFP8 E4M3 row+col cast, 16384x4096 BF16",
        "",
        f"command (FETCH_SIZE): {command.format(counter='FETCH_SIZE')}",
        f"command (WRITE_SIZE): {command.format(counter='WRITE_SIZE')}",
        "",
        f"calibration: torch copy kernel {COPY_KERNEL} moving {COPY_BYTES} B each way reads "
        f"FETCH_SIZE {f['copy']:.1f} KiB (factor {f_cal:.4f}) and WRITE_SIZE {w['copy']:.1f} KiB (factor {w_cal:.4f})",
        f"cast raw: FETCH_SIZE {f['cast']:.1f} KiB, WRITE_SIZE {w['cast']:.1f} KiB per dispatch",
        f"cast fetched bytes per launch (calibrated): {fetch_b:.0f}  (algorithmic read {alg_read}, "
        f"ratio {fetch_b / alg_read:.4f})",
        f"cast written bytes per launch (calibrated): {write_b:.0f}  (algorithmic write {alg_write}, "
        f"ratio {write_b / alg_write:.4f})",
        f"hbm_bytes_per_launch: {fetch_b + write_b:.0f}",
        f"kernel_source_hash: {kernel_hash()}",
    ]
    return "\n".join(lines) + "\n"


def cpu_baseline(x_gpu, budget_s: float = 12.0):
    """The CPU oracle on consecutive 512-row slabs of the same tensor until the
    time budget is used; GB/s on the same algorithmic-byte basis."""
    import mx_inputs as I
    import oracle as O
    slab = 512
    done_rows, t_used = 0, 0.0
    while done_rows < ROWS and t_used < budget_s:
        xs = I.to_bits(x_gpu[done_rows:done_rows + slab])
        t0 = time.perf_counter()
        O.quantize(xs, "bf16", O.E4M3, O.FLOOR, O.BOTH)
        t_used += time.perf_counter() - t0
        done_rows += slab
    nbytes = ALG_BYTES * done_rows / ROWS
    return {"value": round(nbytes / t_used / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first {done_rows} of {ROWS} rows ({done_rows * COLS} elements), fused row+col "
                      f"E4M3 floor, NumPy float64 oracle, single thread, {t_used:.1f} s"}


_PAR_BITS = None


def _oracle_slab(r0):
    """Worker of cpu_baseline_parallel: the oracle on rows r0 .. r0+511 of the
    host copy made before the workers were forked."""
    import oracle as O
    O.quantize(_PAR_BITS[r0:r0 + 512], "bf16", O.E4M3, O.FLOOR, O.BOTH)
    return r0


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_parallel(x_gpu, procs: int):
    """The same oracle over the whole tensor, in `procs` forked worker processes
    taking disjoint 512-row slabs (the workers touch only host memory)."""
    import multiprocessing as mp
    import mx_inputs as I
    global _PAR_BITS
    _PAR_BITS = I.to_bits(x_gpu)
    ctx = mp.get_context("fork")
    with ctx.Pool(procs) as pool:
        pool.map(_oracle_slab, [0])                     # start the workers
        t0 = time.perf_counter()
        pool.map(_oracle_slab, range(0, ROWS, 512), chunksize=1)
        t = time.perf_counter() - t0
    _PAR_BITS = None
    return {"value": round(ALG_BYTES / t / 1e9, 4), "unit": "GB/s", "cores": procs, "kind": "oracle",
            "sample": f"all {ROWS} rows in 512-row slabs over {procs} processes, fused row+col E4M3 floor, "
                      f"NumPy float64 oracle, {t:.2f} s; CPU {_cpu_model()}"}


CODE_BITS = {"e4m3": 8, "e5m2": 8, "e2m1": 4, "e2m3": 6, "e3m2": 6, "int8": 8}


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


def _cast_workload(gen, b, r, c, esize, fmt, mode, axis, desc, rounding="rne", block="1x32"):
    """One quantize launch per step over one tensor; bytes = input + code and scale planes."""
    planes = (2 if axis == "both" else 1)
    per_scale = 32 * 32 if block == "32x32" else 32
    nbytes = b * r * c * esize + planes * (b * r * c * CODE_BITS[fmt] // 8 + b * r * c // per_scale)

    def make(dev, i):
        import microscaling_block_quantized_amd as mx
        x = gen(dev, i).reshape(b, r, c)
        return mx.BoundQuantize(x, fmt, mode, axis, _planes(dev, b, r, c, fmt, axis, block), rounding=rounding,
                                seed=0x5EED + i, block=block)
    cfg = {"workload": desc, "batch": b, "rows": r, "cols": c, "fmt": fmt, "scale_mode": mode, "axis": axis}
    if rounding != "rne" or block != "1x32":
        cfg.update(rounding=rounding, block=block)
    return {"bytes": nbytes, "make": make, "metric": f"GB/s (read+write), {desc}", "config": cfg,
            "dtype": "bf16" if esize == 2 else "f32"}


def _nvfp4_workload():
    """16384x4096 BF16 activations -> NVFP4, both copies, global scale computed
    in the same call (its amax pass reads the input a second time)."""
    b, r, c = 1, ROWS, COLS
    n = b * r * c
    nbytes = 2 * n * 2 + 2 * (n // 2 + n // 16) + 4

    def make(dev, i):
        import torch
        import microscaling_block_quantized_amd as mx
        import mx_inputs as I
        x = I.activations(r, c, seed=1 + i, device=dev).view(b, r, c)
        out = {"global_scale": torch.empty((b,), dtype=torch.float32, device=dev),
               "row_codes": torch.empty((b, r, c // 2), dtype=torch.uint8, device=dev),
               "row_scales": torch.empty((b, r, c // 16), dtype=torch.uint8, device=dev),
               "col_codes": torch.empty((b, c, r // 2), dtype=torch.uint8, device=dev),
               "col_scales": torch.empty((b, c, r // 16), dtype=torch.uint8, device=dev)}
        return mx.BoundQuantizeNvfp4(x, "both", out)
    desc = ("activations 16384x4096 bf16 -> NVFP4 (E2M1, 16-element UE4M3 blocks, FP32 global scale) row+col, "
            "global scale computed in the call")
    return {"bytes": nbytes, "make": make, "metric": f"GB/s (read+write), {desc}", "dtype": "bf16",
            "config": {"workload": desc, "batch": b, "rows": r, "cols": c, "fmt": "nvfp4", "axis": "both",
                       "input_reads": 2}}


def _requant_workload():
    """14336x4096 weights as MXFP4 (E2M1, floor, rows; made once, untimed) ->
    FP8 E4M3 with 128x128 block scales, both the row copy and the transposed
    copy, plus the per-block spread."""
    r, c = 14336, 4096
    n = r * c
    nblk = (r // 128) * (c // 128)
    nbytes = (n // 2 + n // 32) + 2 * (n + 4 * nblk) + nblk

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
        return mx.BoundRequant(q["row_codes"], q["row_scales"], (r, c), "both", out)
    desc = ("weights 14336x4096 as MXFP4 (E2M1 1x32, floor) -> FP8 E4M3 with 128x128 power-of-two block scales, "
            "row copy + transposed copy + scale-spread check")
    # 16 sets: 500 MB of MXFP4 inputs, so none is still in the 256 MB memory-side cache when its turn comes
    return {"bytes": nbytes, "make": make, "metric": f"GB/s (read+write), {desc}", "sets": 16, "dtype": "u8",
            "config": {"workload": desc, "rows": r, "cols": c, "fmt": "e2m1->e4m3", "axis": "both"}}


def _qat_workload():
    """14336x4096 FP32 master weights -> MXFP4 (E2M1 1x32, floor) -> FP8 E4M3 with
    128x128 block scales, one pass: the MXFP4 plane, both FP8 copies and the
    spreads are written."""
    r, c = 14336, 4096
    n = r * c
    nblk = (r // 128) * (c // 128)
    nbytes = 4 * n + (n // 2 + n // 32) + 2 * (n + 4 * nblk) + nblk

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
        return mx.BoundQuantizeFp4Fp8(x, "floor", "both", out)
    desc = ("FP32 master weights 14336x4096 -> MXFP4 (E2M1 1x32, floor) -> FP8 E4M3 with 128x128 power-of-two "
            "block scales in one pass: MXFP4 plane + row copy + transposed copy + spreads")
    return {"bytes": nbytes, "make": make, "metric": f"GB/s (read+write), {desc}", "dtype": "f32",
            "config": {"workload": desc, "rows": r, "cols": c, "fmt": "f32->e2m1->e4m3", "axis": "both"}}


def _wide_range_pipeline():
    """64 x 4096x14336 BF16: fused E4M3 quantize, then both planes dequantized to BF16."""
    b, r, c = 64, 4096, 14336
    n = b * r * c
    nbytes = (n * 2 + 2 * (n + n // 32)) + 2 * (n + n // 32 + n * 2)

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
        return step
    return {"bytes": nbytes, "make": make, "sets": 1, "dtype": "bf16",
            "metric": "GB/s (read+write), 64x4096x14336 BF16 MXFP8 E4M3 row+col quantize + both dequantizes",
            "config": {"workload": "wide-range batch 64x4096x14336 bf16: fused E4M3 quantize (floor), then "
                                   "row and column planes dequantized to bf16",
                       "batch": b, "rows": r, "cols": c, "fmt": "e4m3", "scale_mode": "floor", "axis": "both"}}


def _fp32_normal_round_trip():
    """256x1024 FP32 N(0,1): row-wise E4M3 quantize (floor) + dequantize to FP32."""
    r, c = 256, 1024
    n = r * c
    nbytes = (n * 4 + n + n // 32) + (n + n // 32 + n * 4)

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
        return step
    return {"bytes": nbytes, "make": make, "dtype": "f32",
            "metric": "GB/s (read+write), 256x1024 FP32 MXFP8 E4M3 row quantize + dequantize",
            "config": {"workload": "fp32 N(0,1) 256x1024: row-wise E4M3 quantize (floor) + dequantize to fp32",
                       "rows": r, "cols": c, "fmt": "e4m3", "scale_mode": "floor", "axis": "row"}}


def _gen(name):
    def g(dev, i):
        import mx_inputs as I
        if name == "activations":
            return I.activations(ROWS, COLS, seed=1 + i, device=dev)
        if name == "weights":
            return I.weights(14336, 4096, seed=2 + 100 * i, device=dev)
        if name == "gradients":
            return I.gradients(8192, 8192, seed=3 + 100 * i, device=dev)
        raise KeyError(name)
    return g


WORKLOADS = {
    "activations": _cast_workload(_gen("activations"), 1, ROWS, COLS, 2, "e4m3", "floor", "both",
                                  "activations 16384x4096 bf16 -> MXFP8 E4M3 row+col fused, floor scale rule"),
    "weights_floor": _cast_workload(_gen("weights"), 1, 14336, 4096, 2, "e2m1", "floor", "row",
                                    "weights 14336x4096 bf16 -> MXFP4 E2M1 row-wise, floor scale rule"),
    "weights_roundup": _cast_workload(_gen("weights"), 1, 14336, 4096, 2, "e2m1", "roundup", "row",
                                      "weights 14336x4096 bf16 -> MXFP4 E2M1 row-wise, round-up scale rule"),
    "gradients": _cast_workload(_gen("gradients"), 1, 8192, 8192, 4, "e5m2", "roundup", "col",
                                "gradients 8192x8192 fp32 -> MXFP8 E5M2 column-wise, round-up scale rule"),
    "act_e2m3": _cast_workload(_gen("activations"), 1, ROWS, COLS, 2, "e2m3", "floor", "both",
                               "activations 16384x4096 bf16 -> MXFP6 E2M3 row+col fused, floor scale rule"),
    "act_e3m2": _cast_workload(_gen("activations"), 1, ROWS, COLS, 2, "e3m2", "floor", "both",
                               "activations 16384x4096 bf16 -> MXFP6 E3M2 row+col fused, floor scale rule"),
    "act_int8": _cast_workload(_gen("activations"), 1, ROWS, COLS, 2, "int8", "floor", "both",
                               "activations 16384x4096 bf16 -> MXINT8 row+col fused, floor scale rule"),
    "grad_sr_e2m1": _cast_workload(_gen("gradients"), 1, 8192, 8192, 4, "e2m1", "roundup", "col",
                                   "gradients 8192x8192 fp32 -> MXFP4 E2M1 column-wise, stochastic rounding, "
                                   "round-up scale rule", rounding="sr"),
    "weights_2d_e2m1": _cast_workload(_gen("weights"), 1, 14336, 4096, 2, "e2m1", "floor", "both",
                                      "weights 14336x4096 bf16 -> MXFP4 E2M1 32x32 blocks, row+col fused, "
                                      "floor scale rule", block="32x32"),
    "act_nvfp4": _nvfp4_workload(),
    "weights_fp4_in_fp8": _requant_workload(),
    "qat_fp4_fp8": _qat_workload(),
    "wide_range": _wide_range_pipeline(),
    "fp32_normal": _fp32_normal_round_trip(),
}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=0,
                    help="rotating input/output buffer sets (default per workload: 8; 16 for the "
                         "requantization; 1 for the 30 GB wide-range batch)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-procs", type=int, default=16,
                    help="worker processes of the parallel oracle baseline (0: skip it); capped at the host's cores")
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
    ap.add_argument("--trace-workload", default="activations", choices=sorted(TRACE_KERNELS),
                    help="which workload's kernels --summarize-trace / --summarize-counters report")
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.command, args.trace_workload), end="")
        return 0
    if args.summarize_sq:
        print(summarize_sq(args.command, args.summarize_sq), end="")
        return 0
    if args.summarize_counters:
        if args.trace_workload == "activations":
            print(summarize_counters(*args.summarize_counters, args.command), end="")
        else:
            print(summarize_counters_of(*args.summarize_counters, args.command, args.trace_workload), end="")
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
    steps_fns = [wl["make"](dev, i) for i in range(args.sets)]
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
    del steps_fns
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
    traffic = read_counters() if args.workload == "activations" else None
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
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic},
        "copy_ceiling": {"value": round(copy_gbs, 2), "unit": "GB/s",
                         "what": f"libmx non-temporal 16-byte copy (mx_copy_nt), {copy_half} B each way, "
                                 "3 rotating destinations",
                         "frac_of_ceiling": round(gbs / copy_gbs, 4),
                         "torch_device_copy": round(torch_copy_gbs, 2)},
    }
    ops = valu_ops_per_element(args.workload) if args.workload in ALU_BOUND else None
    if ops is not None:
        # VALU-bound: the roofline is the VALU issue rate; the HBM view stays beside it
        elems = SQ_KERNELS[args.workload][1]
        tops = ops * elems / (ms * 1e-3) / 1e12
        line["hbm_roofline"] = line["roofline"]
        line["roofline"] = {"bound": "alu", "achieved": round(tops, 3), "peak": round(VALU_PEAK_T_LANE_OPS, 2),
                            "unit": "T VALU lane-ops/s", "frac": round(tops / VALU_PEAK_T_LANE_OPS, 4),
                            "traffic": None, "valu_lane_ops_per_element": ops,
                            "source": "profiles/valu_lds_counters.md (SQ_INSTS_VALU x 64 / elements)"}
    if not args.no_cpu_baseline and args.workload == "activations":
        import mx_inputs as I
        xa = I.activations(ROWS, COLS, seed=1, device=dev)
        line["cpu_baseline"] = cpu_baseline(xa)
        procs = min(args.cpu_procs, os.cpu_count() or 1)
        if procs > 1:
            line["cpu_baseline_parallel"] = cpu_baseline_parallel(xa, procs)
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
