"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws and arranges input values; it holds none of the MX
quantization arithmetic, and it is the only code both the HIP-path tests and
the CPU oracle read. Every generator takes a seed and a torch device and is
deterministic for a given (seed, device type).

Workloads (shapes and value distributions of LLM tensors):
  fp32_normal       256x1024 FP32, N(0, 1)
  activations       16384x4096 BF16, N(0, 1) with outlier channels: 4 whole
                    columns (0.1% of 4096, rounded) scaled x100
  weights           14336x4096 BF16, N(0, sigma_r^2) with sigma_r per row
                    log-uniform in [0.005, 0.05]
  gradients         8192x8192 FP32, Student-t(3) * 1e-4, then exactly 1% zeros,
                    0.01% specials (+Inf, -Inf, NaN with equal odds), and 16
                    column blocks plus 16 row blocks of 32 zeroed last
  wide_range        4096x14336 BF16 per tensor, uniform(-1, 1) * 2^k with an
                    integer k uniform in [-20, 20] per 1x32 row block
Directed inputs: an exhaustive BF16 sweep (every BF16 pattern under every
reachable shared scale), an amax sweep (every finite BF16 magnitude as a
block maximum) and hand-picked FP32 edge blocks.
"""
from __future__ import annotations

import math

import torch

__all__ = [
    "fp32_normal", "activations", "weights", "gradients", "wide_range", "wide_range_batch",
    "bf16_sweep", "bf16_amax_sweep", "fp32_edges", "bf16_edges", "to_bits", "FMT_MAX",
]

# Largest finite element magnitude and its binade, used only to place anchor
# values when arranging the sweep inputs.
FMT_MAX = {"e4m3": (448.0, 8), "e5m2": (57344.0, 15), "e2m1": (6.0, 2), "e2m3": (7.5, 2),
           "e3m2": (28.0, 4), "int8": (127 / 64, 0)}
# (mantissa bits, bias) of the sign/exponent/mantissa formats, for placing probes
_FP_LAYOUT = {"e4m3": (3, 7), "e5m2": (2, 15), "e2m3": (3, 1), "e3m2": (2, 3)}


def _gen(seed: int, device) -> torch.Generator:
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    return g


def to_bits(t: torch.Tensor):
    """numpy view of a tensor's raw bits: uint16 for bfloat16, float32 as is."""
    import numpy as np
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def fp32_normal(rows=256, cols=1024, seed=0, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    return torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32)


def activations(rows=16384, cols=4096, seed=1, device="cpu", outlier_frac=0.001, gain=100.0):
    g = _gen(seed, device)
    x = torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32)
    n_out = max(1, round(outlier_frac * cols))
    idx = torch.randperm(cols, generator=g, device=device)[:n_out]
    x[:, idx] *= gain
    return x.to(torch.bfloat16)


def weights(rows=14336, cols=4096, seed=2, device="cpu", lo=0.005, hi=0.05):
    g = _gen(seed, device)
    u = torch.rand((rows, 1), generator=g, device=device, dtype=torch.float64)
    sigma = torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo))).to(torch.float32)
    x = torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32) * sigma
    return x.to(torch.bfloat16)


def gradients(rows=8192, cols=8192, seed=3, device="cpu", scale=1e-4, zero_frac=0.01,
              special_frac=1e-4, zero_col_blocks=16, zero_row_blocks=16):
    g = _gen(seed, device)
    z = torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32)
    chi = torch.randn((3, rows, cols), generator=g, device=device, dtype=torch.float32).square_().sum(0)
    x = z / torch.sqrt(chi / 3.0) * scale            # Student-t with 3 degrees of freedom
    flat = x.view(-1)
    n = flat.numel()
    n_zero = round(zero_frac * n)
    n_spec = round(special_frac * n)
    perm = torch.randperm(n, generator=g, device=device)
    flat[perm[:n_zero]] = 0.0
    spec_idx = perm[n_zero:n_zero + n_spec]
    kind = torch.randint(0, 3, (n_spec,), generator=g, device=device)
    vals = torch.tensor([math.inf, -math.inf, math.nan], device=device, dtype=torch.float32)
    flat[spec_idx] = vals[kind]
    # whole 32-element blocks of exact zeros, written last so they stay pure zero
    if rows >= 32:
        cb = torch.randint(0, rows // 32, (zero_col_blocks,), generator=g, device=device).tolist()
        cc = torch.randint(0, cols, (zero_col_blocks,), generator=g, device=device).tolist()
        for rb, c in zip(cb, cc):
            x[rb * 32:(rb + 1) * 32, c] = 0.0
    if cols >= 32:
        rr = torch.randint(0, rows, (zero_row_blocks,), generator=g, device=device).tolist()
        rc = torch.randint(0, cols // 32, (zero_row_blocks,), generator=g, device=device).tolist()
        for r, cblk in zip(rr, rc):
            x[r, cblk * 32:(cblk + 1) * 32] = 0.0
    return x


def wide_range(index=0, rows=4096, cols=14336, seed=4, device="cpu", kmax=20):
    g = _gen(seed * 1_000_003 + index, device)
    u = torch.rand((rows, cols), generator=g, device=device, dtype=torch.float32) * 2.0 - 1.0
    k = torch.randint(-kmax, kmax + 1, (rows, cols // 32, 1), generator=g, device=device)
    x = u.view(rows, cols // 32, 32) * torch.exp2(k.to(torch.float32))
    return x.view(rows, cols).to(torch.bfloat16)


def wide_range_batch(batch=64, rows=4096, cols=14336, seed=4, device="cpu", kmax=20):
    out = torch.empty((batch, rows, cols), dtype=torch.bfloat16, device=device)
    for i in range(batch):
        out[i] = wide_range(i, rows, cols, seed, device, kmax)
    return out


def _bf16_from_bits(bits: torch.Tensor) -> torch.Tensor:
    return bits.to(torch.int16).view(torch.bfloat16)


def bf16_sweep(fmt: str) -> torch.Tensor:
    """Every finite BF16 pattern under every reachable shared scale, as blocks.

    For each exponent e that a block can take (anchor 2^e * max must be a BF16
    normal), one anchor of magnitude max * 2^e fixes the block scale at e under
    both scale rules, and the other 31 slots hold BF16 patterns of magnitude
    <= anchor, both signs, all of them in turn. The anchor's slot rotates so
    every lane position is exercised. Returns [n_blocks, 32] bfloat16.
    """
    vmax, emax = FMT_MAX[fmt]
    mant_bits = int(round((vmax / 2 ** emax - 1.0) * 128))      # 7-bit significand of max
    chunks = []
    slot = 0
    for field in range(emax - 127 + 127, 255):                   # anchor exponent field
        e = field - 127 - emax
        if e < -127:
            continue
        anchor = (field << 7) | mant_bits
        mags = torch.arange(0, anchor + 1, dtype=torch.int32)
        probes = torch.cat([mags, mags | 0x8000])
        pad = (-probes.numel()) % 31
        if pad:
            probes = torch.cat([probes, torch.zeros(pad, dtype=torch.int32)])
        probes = probes.view(-1, 31)
        nb = probes.shape[0]
        blk = torch.empty((nb, 32), dtype=torch.int32)
        pos = (torch.arange(nb) + slot) % 32
        slot = (slot + nb) % 32
        cols = torch.arange(32).view(1, 32)
        is_anchor = cols == pos.view(-1, 1)
        src = torch.cumsum(~is_anchor, dim=1) - 1                 # probe index for non-anchor slots
        src = src.clamp(min=0)
        blk = torch.where(is_anchor, torch.full_like(blk, anchor), torch.gather(probes, 1, src))
        chunks.append(blk)
    return _bf16_from_bits(torch.cat(chunks))


def bf16_amax_sweep() -> torch.Tensor:
    """One block per finite positive BF16 magnitude m (and zero): slot m % 32
    holds m with sign alternating per block, the others hold m >> 1 (a smaller
    magnitude). Returns [32641, 32] bfloat16."""
    m = torch.arange(0, 0x7F81, dtype=torch.int32)
    m = m[m < 0x7F80]
    small = m >> 1
    blk = small.view(-1, 1).repeat(1, 32)
    pos = m % 32
    sign = (m % 2) << 15
    blk[torch.arange(m.numel()), pos] = m | sign
    return _bf16_from_bits(blk)


def _f32(v) -> torch.Tensor:
    return torch.tensor(v, dtype=torch.float32)


def fp32_edges(fmt: str) -> torch.Tensor:
    """Hand-built FP32 blocks that stress the edges of the cast for `fmt`:
    exact midpoints between adjacent codes and one ulp either side, saturation
    boundaries, FP32 subnormal elements and block maxima, the clamp of the
    scale at 2^-127, zero / signed-zero blocks and blocks holding NaN or Inf.
    Returns [n, 32] float32."""
    vmax, emax = FMT_MAX[fmt]
    blocks = []
    # code grid of the element format (magnitudes), built from its bit layout
    if fmt == "e2m1":
        grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    elif fmt == "int8":
        grid = [k / 64.0 for k in range(128)]
    else:
        mb, bias = _FP_LAYOUT[fmt]
        grid = []
        for code in range(0, 1 << 7):
            ex, man = code >> mb, code & ((1 << mb) - 1)
            val = (man / (1 << mb)) * 2.0 ** (1 - bias) if ex == 0 else (1 + man / (1 << mb)) * 2.0 ** (ex - bias)
            if val <= vmax:
                grid.append(val)
        grid = sorted(set(grid))
    mids = [(a + b) / 2 for a, b in zip(grid[:-1], grid[1:])]
    probes = []
    for v in mids + grid:
        f = torch.tensor(v, dtype=torch.float32)
        probes += [f.item(), torch.nextafter(f, _f32(math.inf)).item(), torch.nextafter(f, _f32(0.0)).item()]
    top = torch.nextafter(_f32(2.0 ** (emax + 1)), _f32(0.0)).item()   # largest value below 2^(emax+1)
    sat = [top, vmax * 1.03, vmax * 1.0625, vmax * 1.07, vmax * 1.125, vmax * 1.5, -vmax * 1.9, vmax,
           -vmax, vmax * 0.999]
    for e in (-127, -126, -120, -100, -20, -3, 0, 5, 40, 100):
        anchor = vmax * 2.0 ** e                 # fixes the block exponent at e under both rules
        p = [x * 2.0 ** e for x in probes]
        for s in (1.0, -1.0):
            row = [s * y for y in p]
            for i in range(0, len(row), 31):
                part = row[i:i + 31]
                part = part + [0.0] * (31 - len(part))
                blocks.append([anchor] + part)
        # elements above max inside a block whose floor exponent is e: they clip
        blocks.append([x * 2.0 ** e for x in sat] + [2.0 ** e] * (32 - len(sat)))
    # FP32 subnormal elements and maxima
    sub = [2.0 ** -149, 3 * 2.0 ** -149, 2.0 ** -140, 1.5 * 2.0 ** -130, 2.0 ** -127, -2.0 ** -133]
    blocks.append(sub + [0.0] * (32 - len(sub)))
    blocks.append([2.0 ** -126] + sub + [-0.0] * (31 - len(sub)))
    blocks.append([1.0] + sub + [2.0 ** -10 * k for k in range(25)])
    # subnormal block maxima whose mantissa field sits around 0x7E0000 and 0x7F0000
    for mant in (0x7E0000, 0x7E0001, 0x7F0000, 0x7F0001, 0x7FFFFF):
        amax = mant * 2.0 ** -149
        blocks.append([amax, -amax] + [amax * k / 32 for k in range(30)])
    # tiny normal maxima around the scale clamp (round-up edge included)
    t = torch.tensor(1.75 * 2.0 ** -119, dtype=torch.float32)
    tn = torch.nextafter(t, _f32(math.inf)).item()
    for amax in (tn, 1.75 * 2.0 ** -119, 1.5 * 2.0 ** -125, 2.0 ** -118, 2.0 ** -119):
        blocks.append([amax] + [amax * (k - 15) / 16 for k in range(31)])
    # near the top of the FP32 range
    big = torch.tensor(3.4028234663852886e38, dtype=torch.float32).item()
    blocks.append([big, -big] + [big / 2 ** k for k in range(30)])
    blocks.append([1.9375 * 2.0 ** 127] + [2.0 ** 120] * 31)
    # zero, signed zero, specials
    blocks.append([0.0] * 32)
    blocks.append([-0.0] * 32)
    blocks.append([-0.0, 0.0] * 16)
    blocks.append([math.nan] + [1.0] * 31)
    blocks.append([1.0] * 31 + [math.inf])
    blocks.append([-math.inf] + [0.0] * 31)
    blocks.append([math.nan] * 32)
    return torch.tensor(blocks, dtype=torch.float32)


def bf16_edges(fmt: str) -> torch.Tensor:
    """fp32_edges rounded to BF16 (inputs only; exactness of the probes is not
    required), plus BF16 subnormal blocks. Returns [n, 32] bfloat16."""
    e = fp32_edges(fmt).to(torch.bfloat16)
    subs = torch.arange(1, 0x80, dtype=torch.int32)             # every BF16 subnormal magnitude
    sub_blocks = torch.cat([subs, subs | 0x8000, torch.zeros(2, dtype=torch.int32)]).view(-1, 32)
    return torch.cat([e, _bf16_from_bits(sub_blocks)])
