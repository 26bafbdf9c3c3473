"""Python binding of libmx (MX block quantization on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libmx.so``. torch provides device memory and the current stream.
The functions mirror the C ABI in ``include/libmx.h``:

    mx_quantize(x, fmt, mode, axis, rounding, seed, block)
                                         -> dict of uint8 code / scale planes
                                            (mx_quantize_ex when rounding or block
                                            is not the default)
    mx_dequantize(codes, scales, fmt, shape, out_dtype, block)
    mx_quantize_nvfp4(x, axis, global_scale) / mx_dequantize_nvfp4(...)
    mx_plane_bytes(fmt, shape, axis)     -> (code bytes, scale bytes) of the planes of `axis`
    mx_strerror(err), mx_version()

There is no CPU path: inputs must be GPU tensors, and a missing ``libmx.so``
raises at the first call. Before any call, every tensor is checked against
the sizes the shape and format imply (dtype, contiguity, byte count, device):
the C ABI trusts the caller's buffer sizes, so a short buffer would otherwise
be written past its end.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "MXError", "FMT", "CODE_BITS", "MODE", "AXIS", "DTYPE", "ROUNDING", "BLOCK", "MxQuantOpts", "lib_path", "load", "mx_version", "mx_strerror",
    "mx_plane_bytes", "mx_quantize", "mx_dequantize", "mx_quantize_nvfp4", "mx_dequantize_nvfp4",
    "mx_requant_fp4_fp8", "mx_quantize_fp4_fp8", "mx_copy_nt", "EXPORTS", "BoundQuantize", "BoundDequantize",
    "BoundQuantizeNvfp4", "BoundRequant", "BoundQuantizeFp4Fp8",
]

FMT = {"e4m3": 0, "e5m2": 1, "e2m1": 2, "e2m3": 3, "e3m2": 4, "int8": 5}
CODE_BITS = {"e4m3": 8, "e5m2": 8, "e2m1": 4, "e2m3": 6, "e3m2": 6, "int8": 8}
MODE = {"floor": 0, "roundup": 1}
AXIS = {"row": 1, "col": 2, "both": 3}
ROUNDING = {"rne": 0, "sr": 1}
BLOCK = {"1x32": 0, "32x32": 1}
DTYPE = {"f32": 0, "bf16": 1}
EXPORTS = ("mx_plane_bytes", "mx_quantize", "mx_quantize_ex", "mx_dequantize", "mx_dequantize_ex",
           "mx_quantize_nvfp4", "mx_dequantize_nvfp4", "mx_requant_fp4_fp8", "mx_quantize_fp4_fp8", "mx_copy_nt",
           "mx_strerror", "mx_version")

_LIB = None


class MXError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: libmx error {code}: {mx_strerror(code)}")
        self.code = code


class MxShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


class MxQuantOpts(ctypes.Structure):
    _fields_ = [("rounding", ctypes.c_int), ("block", ctypes.c_int), ("seed", ctypes.c_uint64)]


def lib_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmx.so")


def load() -> ctypes.CDLL:
    """Load libmx.so (built by ``python -m microscaling_block_quantized_amd.build``)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"libmx.so not built at {path}; run "
                           "`python -m microscaling_block_quantized_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, u8p = ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p
    lib.mx_version.restype = i32
    lib.mx_version.argtypes = []
    lib.mx_strerror.restype = ctypes.c_char_p
    lib.mx_strerror.argtypes = [i32]
    lib.mx_plane_bytes.restype = i32
    lib.mx_plane_bytes.argtypes = [i32, MxShape, i32, ctypes.POINTER(ctypes.c_size_t),
                                   ctypes.POINTER(ctypes.c_size_t)]
    lib.mx_quantize.restype = i32
    lib.mx_quantize.argtypes = [vp, i32, MxShape, i32, i32, i32, vp, u8p, vp, u8p, vp]
    lib.mx_dequantize.restype = i32
    lib.mx_dequantize.argtypes = [vp, u8p, i32, MxShape, i32, vp, vp]
    lib.mx_quantize_ex.restype = i32
    lib.mx_quantize_ex.argtypes = [vp, i32, MxShape, i32, i32, i32, ctypes.POINTER(MxQuantOpts), vp, u8p, vp,
                                   u8p, vp]
    lib.mx_dequantize_ex.restype = i32
    lib.mx_dequantize_ex.argtypes = [vp, u8p, i32, MxShape, i32, i32, vp, vp]
    lib.mx_quantize_nvfp4.restype = i32
    lib.mx_quantize_nvfp4.argtypes = [vp, i32, MxShape, i32, vp, i32, vp, u8p, vp, u8p, vp]
    lib.mx_dequantize_nvfp4.restype = i32
    lib.mx_dequantize_nvfp4.argtypes = [vp, u8p, vp, MxShape, i32, vp, vp]
    lib.mx_requant_fp4_fp8.restype = i32
    lib.mx_requant_fp4_fp8.argtypes = [vp, u8p, MxShape, i32, u8p, vp, u8p, vp, u8p, vp]
    lib.mx_quantize_fp4_fp8.restype = i32
    lib.mx_quantize_fp4_fp8.argtypes = [vp, i32, MxShape, i32, i32, vp, u8p, u8p, vp, u8p, vp, u8p, vp]
    lib.mx_copy_nt.restype = i32
    lib.mx_copy_nt.argtypes = [vp, vp, ctypes.c_int64, vp]
    _LIB = lib
    return lib


def mx_version() -> int:
    return load().mx_version()


def mx_strerror(err: int) -> str:
    return load().mx_strerror(int(err)).decode()


def mx_copy_nt(src, dst) -> None:
    """Copy GPU tensor src into dst (same byte size, a multiple of 16) with the
    library's plain non-temporal copy kernel: the bandwidth ceiling the casts
    are measured against, not an MX operation."""
    if not (src.is_cuda and dst.is_cuda):
        raise ValueError("mx_copy_nt needs GPU tensors (libmx has no CPU path)")
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n or not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("mx_copy_nt needs contiguous tensors of the same byte size")
    import torch
    with torch.cuda.device(src.device):
        err = load().mx_copy_nt(_ptr(src), _ptr(dst), n, _stream_of(src))
    if err:
        raise MXError(err, "mx_copy_nt")


def _shape3(shape) -> tuple:
    shape = tuple(int(v) for v in shape)
    if len(shape) == 2:
        return (1,) + shape
    if len(shape) != 3:
        raise ValueError(f"expected a 2-D or 3-D shape, got {shape}")
    return shape


def mx_plane_bytes(fmt: str, shape, axis: str = "row") -> tuple:
    """(code bytes, scale bytes) summed over the planes of `axis` (1x32 blocks)."""
    b, r, c = _shape3(shape)
    cb, sb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    err = load().mx_plane_bytes(FMT[fmt], MxShape(b, r, c), AXIS[axis], ctypes.byref(cb), ctypes.byref(sb))
    if err:
        raise MXError(err, "mx_plane_bytes")
    return cb.value, sb.value


def _check(t, name: str, nbytes: int, dtype, dev) -> None:
    """Raise ValueError unless t is a contiguous tensor of `dtype` on `dev`
    holding exactly `nbytes` bytes."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}; expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    got = t.numel() * t.element_size()
    if got != nbytes:
        raise ValueError(f"{name} holds {got} bytes; this shape and format need {nbytes}")
    if t.device != dev:
        raise ValueError(f"{name} is on {t.device}, the input on {dev}")


def _need_gpu(t, where: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{where} needs GPU tensors (libmx has no CPU path)")


def _input(x, where: str):
    """The input tensor's dtype code after the checks every cast makes."""
    import torch
    if not isinstance(x, torch.Tensor) or x.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"{where}: the input must be a bfloat16 or float32 tensor")
    if not x.is_contiguous():
        raise ValueError(f"{where}: the input must be contiguous")
    return DTYPE["bf16" if x.dtype == torch.bfloat16 else "f32"]


def _mx_plane_shapes(b, r, c, fmt: str, block: str) -> dict:
    """Shapes of the four MX planes of a [b][r][c] tensor. For every shape the
    C ABI accepts they hold exactly the bytes it writes; for any other shape
    the C ABI rejects the call before touching a buffer."""
    bits = CODE_BITS[fmt]
    two = block == "32x32"
    return {"row_codes": (b, r, c * bits // 8),
            "row_scales": (b, max(r // 32, 1), c // 32) if two else (b, r, c // 32),
            "col_codes": (b, c, r * bits // 8),
            "col_scales": (b, c // 32, max(r // 32, 1)) if two else (b, c, max(r // 32, 1))}


def _numel(shape) -> int:
    n = 1
    for v in shape:
        n *= v
    return n


def _check_mx_planes(planes: dict, b, r, c, fmt: str, block: str, dev) -> None:
    import torch
    for k, shp in _mx_plane_shapes(b, r, c, fmt, block).items():
        if k in planes:
            _check(planes[k], k, _numel(shp), torch.uint8, dev)


def _stream_of(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(None)


def _opts(rounding: str, seed: int, block: str):
    if rounding == "rne" and block == "1x32":
        return None
    return MxQuantOpts(ROUNDING[rounding], BLOCK[block], int(seed) & ((1 << 64) - 1))


def mx_quantize(x, fmt: str = "e4m3", mode: str = "floor", axis: str = "both", out: dict | None = None,
                rounding: str = "rne", seed: int = 0, block: str = "1x32"):
    """Quantize a GPU tensor [R][C] or [B][R][C] (bfloat16 or float32).

    Returns {"row_codes", "row_scales"} and/or {"col_codes", "col_scales"} as
    uint8 tensors: row planes [B][R][C'] / [B][R][C/32], column planes
    [B][C][R'] / [B][C][R/32] (C' = C * code bits / 8: C for the 8-bit
    formats, 3C/4 for e2m3 / e3m2, C/2 for e2m1); the batch axis is dropped
    for a 2-D input. ``out`` may supply preallocated planes. rounding "sr"
    (stochastic, with ``seed``) and block "32x32" (scales [B][R/32][C/32] and
    [B][C/32][R/32]) go through mx_quantize_ex.
    """
    import torch
    xdt = _input(x, "mx_quantize")
    b, r, c = _shape3(x.shape)
    squeeze = x.dim() == 2
    ax = AXIS[axis]
    out = out or {}
    dev = x.device

    def plane(name, shp):
        t = out.get(name)
        return t if t is not None else torch.empty(shp, dtype=torch.uint8, device=dev)

    opts = _opts(rounding, seed, block)
    shapes = _mx_plane_shapes(b, r, c, fmt, block)
    planes = {}
    for k in (("row_codes", "row_scales") if ax & 1 else ()) + (("col_codes", "col_scales") if ax & 2 else ()):
        planes[k] = plane(k, shapes[k])
    _check_mx_planes(planes, b, r, c, fmt, block, dev)
    _need_gpu(x, "mx_quantize")
    args = (_ptr(x), xdt, MxShape(b, r, c), FMT[fmt], MODE[mode], ax)
    outs = (_ptr(planes.get("row_codes")), _ptr(planes.get("row_scales")), _ptr(planes.get("col_codes")),
            _ptr(planes.get("col_scales")), _stream_of(x))
    with torch.cuda.device(dev):
        if opts is None:
            err = load().mx_quantize(*args, *outs)
        else:
            err = load().mx_quantize_ex(*args, ctypes.byref(opts), *outs)
    if err:
        raise MXError(err, "mx_quantize_ex" if opts is not None else "mx_quantize")
    if squeeze:
        planes = {k: v[0] for k, v in planes.items()}
    return planes


def mx_dequantize(codes, scales, fmt: str, shape, out_dtype: str = "f32", out=None, block: str = "1x32"):
    """Dequantize one plane; ``shape`` is the element shape of the plane as stored
    (blocks of 32 along its last axis, or 32x32 tiles with block "32x32").
    Returns a float32 or bfloat16 GPU tensor."""
    import torch
    b, r, c = _shape3(shape)
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[out_dtype]
    dev = codes.device
    shp = _mx_plane_shapes(b, r, c, fmt, block)
    _check(codes, "codes", _numel(shp["row_codes"]), torch.uint8, dev)
    _check(scales, "scales", _numel(shp["row_scales"]), torch.uint8, dev)
    y = out if out is not None else torch.empty(tuple(shape), dtype=tdt, device=dev)
    _check(y, "out", b * r * c * (2 if out_dtype == "bf16" else 4), tdt, dev)
    _need_gpu(codes, "mx_dequantize")
    with torch.cuda.device(codes.device):
        if block == "1x32":
            err = load().mx_dequantize(_ptr(codes), _ptr(scales), FMT[fmt], MxShape(b, r, c), DTYPE[out_dtype],
                                       _ptr(y), _stream_of(codes))
        else:
            err = load().mx_dequantize_ex(_ptr(codes), _ptr(scales), FMT[fmt], MxShape(b, r, c), BLOCK[block],
                                          DTYPE[out_dtype], _ptr(y), _stream_of(codes))
    if err:
        raise MXError(err, "mx_dequantize")
    return y


class BoundQuantize:
    """An mx_quantize call with its arguments marshalled once, for repeated
    launches over fixed buffers (benchmark loops). Calling it enqueues one
    quantize on the stream that was current at construction."""

    def __init__(self, x, fmt: str, mode: str, axis: str, out: dict, rounding: str = "rne", seed: int = 0,
                 block: str = "1x32"):
        b, r, c = _shape3(x.shape)
        xdt = _input(x, "BoundQuantize")
        ax = AXIS[axis]
        names = (("row_codes", "row_scales") if ax & 1 else ()) + (("col_codes", "col_scales") if ax & 2 else ())
        if set(k for k, v in out.items() if v is not None) != set(names):
            raise ValueError(f"BoundQuantize: out must hold exactly {names}")
        _check_mx_planes(out, b, r, c, fmt, block, x.device)
        _need_gpu(x, "BoundQuantize")
        head = (_ptr(x), xdt, MxShape(b, r, c), FMT[fmt], MODE[mode], ax)
        tail = (_ptr(out.get("row_codes")), _ptr(out.get("row_scales")), _ptr(out.get("col_codes")),
                _ptr(out.get("col_scales")), _stream_of(x))
        self._opts = _opts(rounding, seed, block)
        if self._opts is None:
            self._fn = load().mx_quantize
            self._args = head + tail
        else:
            self._fn = load().mx_quantize_ex
            self._args = head + (ctypes.byref(self._opts),) + tail
        self._keep = (x, out)

    def __call__(self) -> None:
        err = self._fn(*self._args)
        if err:
            raise MXError(err, "mx_quantize")


class BoundDequantize:
    """An mx_dequantize call with its arguments marshalled once (see BoundQuantize)."""

    def __init__(self, codes, scales, fmt: str, shape, y):
        import torch
        b, r, c = _shape3(shape)
        dev = codes.device
        shp = _mx_plane_shapes(b, r, c, fmt, "1x32")
        _check(codes, "codes", _numel(shp["row_codes"]), torch.uint8, dev)
        _check(scales, "scales", _numel(shp["row_scales"]), torch.uint8, dev)
        if y.dtype not in (torch.bfloat16, torch.float32):
            raise ValueError("BoundDequantize: y must be bfloat16 or float32")
        _check(y, "y", b * r * c * y.element_size(), y.dtype, dev)
        _need_gpu(codes, "BoundDequantize")
        self._fn = load().mx_dequantize
        self._args = (_ptr(codes), _ptr(scales), FMT[fmt], MxShape(b, r, c),
                      DTYPE["bf16" if y.dtype == torch.bfloat16 else "f32"], _ptr(y), _stream_of(codes))
        self._keep = (codes, scales, y)

    def __call__(self) -> None:
        err = self._fn(*self._args)
        if err:
            raise MXError(err, "mx_dequantize")


def _nv_planes(x, axis: str, out: dict | None):
    import torch
    b, r, c = _shape3(x.shape)
    ax = AXIS[axis]
    out = out or {}
    dev = x.device

    def plane(name, shp, dt=torch.uint8):
        t = out.get(name)
        return t if t is not None else torch.empty(shp, dtype=dt, device=dev)

    planes = {"global_scale": plane("global_scale", (b,), torch.float32)}
    if ax & 1:
        planes["row_codes"] = plane("row_codes", (b, r, c // 2))
        planes["row_scales"] = plane("row_scales", (b, r, c // 16))
    if ax & 2:
        planes["col_codes"] = plane("col_codes", (b, c, r // 2))
        planes["col_scales"] = plane("col_scales", (b, c, max(r // 16, 1)))
    return planes


def _check_nv_planes(planes: dict, b, r, c, dev) -> None:
    import torch
    _check(planes["global_scale"], "global_scale", 4 * b, torch.float32, dev)
    for k, nb in (("row_codes", b * r * (c // 2)), ("row_scales", b * r * (c // 16)),
                  ("col_codes", b * c * (r // 2)), ("col_scales", b * c * max(r // 16, 1))):
        if k in planes:
            _check(planes[k], k, nb, torch.uint8, dev)


def mx_quantize_nvfp4(x, axis: str = "both", global_scale=None, out: dict | None = None):
    """NVFP4 cast of a GPU tensor [R][C] or [B][R][C] (bfloat16 or float32).

    Returns {"global_scale" [B] float32, "row_codes" [B][R][C/2], "row_scales"
    [B][R][C/16], "col_codes" [B][C][R/2], "col_scales" [B][C][R/16]} (planes of
    the requested axes; batch axis dropped for a 2-D input, except in
    global_scale). A given ``global_scale`` tensor is used as is instead of the
    tensor's own amax / (6 * 448).
    """
    import torch
    xdt = _input(x, "mx_quantize_nvfp4")
    b, r, c = _shape3(x.shape)
    out = dict(out or {})
    given = global_scale is not None
    if given:
        out["global_scale"] = global_scale
    planes = _nv_planes(x, axis, out)
    _check_nv_planes(planes, b, r, c, x.device)
    _need_gpu(x, "mx_quantize_nvfp4")
    with torch.cuda.device(x.device):
        err = load().mx_quantize_nvfp4(
            _ptr(x), xdt, MxShape(b, r, c), AXIS[axis],
            _ptr(planes["global_scale"]), int(given), _ptr(planes.get("row_codes")), _ptr(planes.get("row_scales")),
            _ptr(planes.get("col_codes")), _ptr(planes.get("col_scales")), _stream_of(x))
    if err:
        raise MXError(err, "mx_quantize_nvfp4")
    if x.dim() == 2:
        planes = {k: (v if k == "global_scale" else v[0]) for k, v in planes.items()}
    return planes


def mx_dequantize_nvfp4(codes, scales, global_scale, shape, out_dtype: str = "f32", out=None):
    """Dequantize one NVFP4 plane; ``shape`` is its element shape as stored."""
    import torch
    b, r, c = _shape3(shape)
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[out_dtype]
    dev = codes.device
    n = b * r * c
    _check(codes, "codes", b * r * (c // 2), torch.uint8, dev)
    _check(scales, "scales", b * r * (c // 16), torch.uint8, dev)
    _check(global_scale, "global_scale", 4 * b, torch.float32, dev)
    y = out if out is not None else torch.empty(tuple(shape), dtype=tdt, device=dev)
    _check(y, "out", n * (2 if out_dtype == "bf16" else 4), tdt, dev)
    _need_gpu(codes, "mx_dequantize_nvfp4")
    with torch.cuda.device(codes.device):
        err = load().mx_dequantize_nvfp4(_ptr(codes), _ptr(scales), _ptr(global_scale), MxShape(b, r, c),
                                         DTYPE[out_dtype], _ptr(y), _stream_of(codes))
    if err:
        raise MXError(err, "mx_dequantize_nvfp4")
    return y


class BoundQuantizeNvfp4:
    """An mx_quantize_nvfp4 call marshalled once (see BoundQuantize)."""

    def __init__(self, x, axis: str, out: dict, global_given: bool = False):
        b, r, c = _shape3(x.shape)
        xdt = _input(x, "BoundQuantizeNvfp4")
        _check_nv_planes(out, b, r, c, x.device)
        _need_gpu(x, "BoundQuantizeNvfp4")
        self._fn = load().mx_quantize_nvfp4
        self._args = (_ptr(x), xdt, MxShape(b, r, c), AXIS[axis],
                      _ptr(out["global_scale"]), int(global_given), _ptr(out.get("row_codes")),
                      _ptr(out.get("row_scales")), _ptr(out.get("col_codes")), _ptr(out.get("col_scales")),
                      _stream_of(x))
        self._keep = (x, out)

    def __call__(self) -> None:
        err = self._fn(*self._args)
        if err:
            raise MXError(err, "mx_quantize_nvfp4")


def _rq_planes(codes, shape, axis: str, spread: bool, out: dict | None):
    import torch
    b, r, c = _shape3(shape)
    nbr, nbc = -(-r // 128), -(-c // 128)
    dev = codes.device
    out = dict(out or {})
    lead = (b,) if len(shape) == 3 else ()
    if AXIS[axis] & 1:
        out.setdefault("e4m3", torch.empty(lead + (r, c), dtype=torch.uint8, device=dev))
        out.setdefault("block_scale", torch.empty(lead + (nbr, nbc), dtype=torch.float32, device=dev))
    if AXIS[axis] & 2:
        out.setdefault("e4m3_t", torch.empty(lead + (c, r), dtype=torch.uint8, device=dev))
        out.setdefault("block_scale_t", torch.empty(lead + (nbc, nbr), dtype=torch.float32, device=dev))
    if spread:
        out.setdefault("spread", torch.empty(lead + (nbr, nbc), dtype=torch.uint8, device=dev))
    return out


def _check_rq_planes(planes: dict, b, r, c, dev) -> None:
    import torch
    n = b * r * c
    nblk = b * (-(-r // 128)) * (-(-c // 128))
    sizes = {"e4m3": (n, torch.uint8), "e4m3_t": (n, torch.uint8), "block_scale": (4 * nblk, torch.float32),
             "block_scale_t": (4 * nblk, torch.float32), "spread": (nblk, torch.uint8),
             "fp4_codes": (b * r * (c // 2), torch.uint8), "fp4_scales": (b * r * (c // 32), torch.uint8)}
    for k, t in planes.items():
        if k not in sizes:
            raise ValueError(f"unknown output plane {k!r}")
        if t is not None:
            _check(t, k, sizes[k][0], sizes[k][1], dev)


def _check_mxfp4_source(codes, scales, b, r, c) -> None:
    import torch
    _check(codes, "codes", b * r * (c // 2), torch.uint8, codes.device)
    _check(scales, "scales", b * r * (c // 32), torch.uint8, codes.device)


def mx_requant_fp4_fp8(codes, scales, shape, axis: str = "row", spread: bool = True, out: dict | None = None):
    """FP4-in-FP8 requantization of an MXFP4 plane (codes [..][R][C/2], scales
    [..][R][C/32] as mx_quantize writes them; ``shape`` is its element shape
    [R][C] or [B][R][C]).

    Returns {"e4m3" [..][R][C], "block_scale" [..][R'][C'] float32} for the row
    axis, {"e4m3_t" [..][C][R], "block_scale_t" [..][C'][R']} for the column axis,
    and "spread" [..][R'][C'] (largest minus smallest active scale code of each
    128x128 block; the block converted exactly when it is at most 14).
    """
    import torch
    b, r, c = _shape3(shape)
    _check_mxfp4_source(codes, scales, b, r, c)
    planes = _rq_planes(codes, shape, axis, spread, out)
    _check_rq_planes(planes, b, r, c, codes.device)
    _need_gpu(codes, "mx_requant_fp4_fp8")
    with torch.cuda.device(codes.device):
        err = load().mx_requant_fp4_fp8(
            _ptr(codes), _ptr(scales), MxShape(b, r, c), AXIS[axis], _ptr(planes.get("e4m3")),
            _ptr(planes.get("block_scale")), _ptr(planes.get("e4m3_t")), _ptr(planes.get("block_scale_t")),
            _ptr(planes.get("spread")), _stream_of(codes))
    if err:
        raise MXError(err, "mx_requant_fp4_fp8")
    return planes


class BoundRequant:
    """An mx_requant_fp4_fp8 call marshalled once (see BoundQuantize)."""

    def __init__(self, codes, scales, shape, axis: str, out: dict):
        b, r, c = _shape3(shape)
        _check_mxfp4_source(codes, scales, b, r, c)
        _check_rq_planes(out, b, r, c, codes.device)
        _need_gpu(codes, "BoundRequant")
        self._fn = load().mx_requant_fp4_fp8
        self._args = (_ptr(codes), _ptr(scales), MxShape(b, r, c), AXIS[axis], _ptr(out.get("e4m3")),
                      _ptr(out.get("block_scale")), _ptr(out.get("e4m3_t")), _ptr(out.get("block_scale_t")),
                      _ptr(out.get("spread")), _stream_of(codes))
        self._keep = (codes, scales, out)

    def __call__(self) -> None:
        err = self._fn(*self._args)
        if err:
            raise MXError(err, "mx_requant_fp4_fp8")


def mx_quantize_fp4_fp8(x, mode: str = "floor", axis: str = "both", fp4: bool = True, spread: bool = True,
                        out: dict | None = None):
    """Master weights x (GPU, bfloat16 or float32, [R][C] or [B][R][C]) ->
    MXFP4 (E2M1, 1x32, scale rule ``mode``) -> FP8 with 128x128 block scales, in
    one pass. Returns the planes of mx_requant_fp4_fp8 plus, with ``fp4``,
    "fp4_codes" [..][R][C/2] and "fp4_scales" [..][R][C/32]."""
    import torch
    xdt = _input(x, "mx_quantize_fp4_fp8")
    b, r, c = _shape3(x.shape)
    planes = _rq_planes(x, tuple(x.shape), axis, spread, out)
    if fp4:
        lead = (b,) if x.dim() == 3 else ()
        planes.setdefault("fp4_codes", torch.empty(lead + (r, c // 2), dtype=torch.uint8, device=x.device))
        planes.setdefault("fp4_scales", torch.empty(lead + (r, c // 32), dtype=torch.uint8, device=x.device))
    _check_rq_planes(planes, b, r, c, x.device)
    _need_gpu(x, "mx_quantize_fp4_fp8")
    with torch.cuda.device(x.device):
        err = load().mx_quantize_fp4_fp8(
            _ptr(x), xdt, MxShape(b, r, c), MODE[mode], AXIS[axis],
            _ptr(planes.get("fp4_codes")), _ptr(planes.get("fp4_scales")), _ptr(planes.get("e4m3")),
            _ptr(planes.get("block_scale")), _ptr(planes.get("e4m3_t")), _ptr(planes.get("block_scale_t")),
            _ptr(planes.get("spread")), _stream_of(x))
    if err:
        raise MXError(err, "mx_quantize_fp4_fp8")
    return planes


class BoundQuantizeFp4Fp8:
    """An mx_quantize_fp4_fp8 call marshalled once (see BoundQuantize)."""

    def __init__(self, x, mode: str, axis: str, out: dict):
        b, r, c = _shape3(x.shape)
        xdt = _input(x, "BoundQuantizeFp4Fp8")
        _check_rq_planes(out, b, r, c, x.device)
        _need_gpu(x, "BoundQuantizeFp4Fp8")
        self._fn = load().mx_quantize_fp4_fp8
        self._args = (_ptr(x), xdt, MxShape(b, r, c), MODE[mode],
                      AXIS[axis], _ptr(out.get("fp4_codes")), _ptr(out.get("fp4_scales")), _ptr(out.get("e4m3")),
                      _ptr(out.get("block_scale")), _ptr(out.get("e4m3_t")), _ptr(out.get("block_scale_t")),
                      _ptr(out.get("spread")), _stream_of(x))
        self._keep = (x, out)

    def __call__(self) -> None:
        err = self._fn(*self._args)
        if err:
            raise MXError(err, "mx_quantize_fp4_fp8")
