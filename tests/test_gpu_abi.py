"""C ABI behaviour on the GPU: streams, guard bands around outputs, reuse of
output buffers, and errors that only a real device can reach."""
import numpy as np
import pytest
import torch

import mx_inputs as I
import oracle as O

pytestmark = pytest.mark.gpu

GUARD = 4096
CANARY = 0xA5


def guarded(nbytes):
    buf = torch.full((nbytes + 2 * GUARD,), CANARY, dtype=torch.uint8, device="cuda")
    return buf, buf[GUARD:GUARD + nbytes]


OFMT = {"e4m3": O.E4M3, "e2m1": O.E2M1, "e2m3": O.E2M3, "e3m2": O.E3M2, "int8": O.INT8}


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1", "e2m3", "e3m2", "int8"])
@pytest.mark.parametrize("shape", [(160, 96), (2, 96, 224), (1, 33, 64), (64, 32)])
def test_writes_stay_inside_outputs(mx, fmt, shape):
    """Every output plane sits between 4 KiB canary bands that must survive."""
    x = torch.randn(shape, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).cuda()
    b, r, c = (1,) + tuple(shape) if len(shape) == 2 else shape
    axis = "both" if r % 32 == 0 else "row"
    bits = OFMT[fmt].bits
    sizes = {"row_codes": (b, r, c * bits // 8), "row_scales": (b, r, c // 32),
             "col_codes": (b, c, r * bits // 8), "col_scales": (b, c, max(r // 32, 1))}
    keys = ["row_codes", "row_scales"] + (["col_codes", "col_scales"] if axis == "both" else [])
    bufs, out = {}, {}
    for k in keys:
        n = int(np.prod(sizes[k]))
        bufs[k], view = guarded(n)
        out[k] = view.view(sizes[k])
    mx.mx_quantize(x.view(b, r, c), fmt, "floor", axis, out=out)
    torch.cuda.synchronize()
    ref = O.quantize(I.to_bits(x.view(b, r, c).cpu()), "bf16", OFMT[fmt],
                     O.FLOOR, O.BOTH if axis == "both" else O.ROW)
    for k in keys:
        buf = bufs[k].cpu().numpy()
        assert (buf[:GUARD] == CANARY).all() and (buf[-GUARD:] == CANARY).all(), k
        assert np.array_equal(out[k].cpu().numpy(), ref[k]), k


@pytest.mark.parametrize("fmt", ["e4m3", "e2m3"])
def test_dequant_writes_stay_inside_output(mx, fmt):
    nbytes = 64 * OFMT[fmt].bits // 8
    codes = torch.randint(0, 256, (96, nbytes), dtype=torch.uint8, generator=torch.Generator().manual_seed(1))
    cbuf, cview = guarded(96 * nbytes)               # codes end right at a canary band
    cview.copy_(codes.view(-1).cuda())
    scales = torch.full((96, 2), 120, dtype=torch.uint8, device="cuda")
    buf, view = guarded(96 * 64 * 2)
    y = view.view(torch.bfloat16).view(96, 64)
    mx.mx_dequantize(cview.view(96, nbytes), scales, fmt, (96, 64), "bf16", out=y)
    torch.cuda.synchronize()
    b = buf.cpu().numpy()
    assert (b[:GUARD] == CANARY).all() and (b[-GUARD:] == CANARY).all()
    ref = O.dequantize(codes.numpy(), scales.cpu().numpy(), OFMT[fmt], "bf16")
    assert np.array_equal(y.cpu().view(torch.int16).numpy().view(np.uint16), ref)


def test_runs_on_the_callers_stream(mx):
    x = I.activations(512, 256, seed=3, device="cuda")
    ref = mx.mx_quantize(x, "e4m3", "floor", "both")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        # the work is enqueued on s; the result is only read after s is synchronized
        out = mx.mx_quantize(x, "e4m3", "floor", "both")
    s.synchronize()
    for k in ref:
        assert torch.equal(ref[k], out[k]), k


def test_output_buffers_can_be_reused(mx):
    a = I.activations(256, 256, seed=4, device="cuda")
    b = I.activations(256, 256, seed=5, device="cuda")
    out = mx.mx_quantize(a, "e5m2", "roundup", "both")
    first = {k: v.clone() for k, v in out.items()}
    mx.mx_quantize(b, "e5m2", "roundup", "both", out=out)
    fresh = mx.mx_quantize(b, "e5m2", "roundup", "both")
    torch.cuda.synchronize()
    for k in out:
        assert torch.equal(out[k], fresh[k])
    assert any(not torch.equal(first[k], out[k]) for k in out)


def test_device_argument_errors(mx):
    x = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mx.MXError) as e:
        mx.mx_quantize(x[:, :48].contiguous(), "e4m3", "floor", "row")
    assert e.value.code == -2
    raw = torch.zeros(64 * 64 + 16, dtype=torch.uint8, device="cuda")
    misaligned = raw[1:1 + 64 * 64].view(64, 64)         # one byte past a 16-byte boundary
    with pytest.raises(mx.MXError) as e:
        mx.mx_quantize(x, "e4m3", "floor", "row", out={"row_codes": misaligned})
    assert e.value.code == -3


def test_copy_nt(mx):
    """The plain non-temporal copy: every byte copied, nothing written outside
    the destination, on the caller's stream."""
    g = torch.Generator(device="cuda").manual_seed(7)
    for nbytes in (16, 4096, 4096 * 257 + 48, 64 << 20):
        src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
        buf, dst = guarded(nbytes)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            mx.mx_copy_nt(src, dst)
        s.synchronize()
        assert torch.equal(dst, src), nbytes
        host = buf.cpu().numpy()
        assert (host[:GUARD] == CANARY).all() and (host[GUARD + nbytes:] == CANARY).all()


def test_graph_capture_and_replay(mx):
    """The library's calls enqueue plain kernels on the caller's stream (no
    allocation, no memset, no synchronization), so a HIP graph can capture a
    quantize + dequantize round trip. The graph is replayed several times with
    new input written eagerly between replays, and every replay is checked
    against the eager calls on the same input."""
    r, c = 256, 1024
    x = torch.empty((1, r, c), dtype=torch.float32, device="cuda")
    planes = {"row_codes": torch.empty((1, r, c), dtype=torch.uint8, device="cuda"),
              "row_scales": torch.empty((1, r, c // 32), dtype=torch.uint8, device="cuda")}
    y = torch.empty((1, r, c), dtype=torch.float32, device="cuda")

    def round_trip():
        mx.mx_quantize(x, "e4m3", "floor", "row", out=planes)
        mx.mx_dequantize(planes["row_codes"], planes["row_scales"], "e4m3", (1, r, c), "f32", out=y)

    x.copy_(I.fp32_normal(r, c, seed=100, device="cuda").view(1, r, c))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        round_trip()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        round_trip()
    torch.cuda.synchronize()
    for k in range(4):
        xin = I.fp32_normal(r, c, seed=200 + k, device="cuda").view(1, r, c) * (2.0 ** (8 * k - 12))
        x.copy_(xin)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {"codes": planes["row_codes"].clone(), "scales": planes["row_scales"].clone(), "y": y.clone()}
        ref = mx.mx_quantize(xin.contiguous(), "e4m3", "floor", "row")
        yref = mx.mx_dequantize(ref["row_codes"], ref["row_scales"], "e4m3", (1, r, c), "f32")
        torch.cuda.synchronize()
        assert torch.equal(got["codes"], ref["row_codes"]), k
        assert torch.equal(got["scales"], ref["row_scales"]), k
        assert torch.equal(got["y"].view(torch.int32), yref.view(torch.int32)), k
