"""The C ABI on the host: exported symbols, plane sizes and argument errors.

None of these calls reaches a GPU: every call here fails validation, which
returns before the first HIP call. The addresses are fake, so a call that
passed validation would launch a kernel on them; to show that a check lets a
case through, a test makes a later check fail instead (an alias, or an
oversized extent).
"""
import ctypes
import os
import re

import pytest

import microscaling_block_quantized_amd as mxb
from microscaling_block_quantized_amd import MxShape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MX_OK, E_NULL, E_SHAPE, E_ALIGN, E_ENUM, E_ALIAS, E_BIG, E_LAUNCH = 0, -1, -2, -3, -4, -5, -6, -7


def declared_functions():
    text = open(os.path.join(ROOT, "include", "libmx.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(mx_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return mxb.load()


def test_library_exports_every_declared_function(lib):
    names = declared_functions()
    assert names == sorted(mxb.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strerror(lib):
    assert mxb.mx_version() == 10700
    for code in (MX_OK, E_NULL, E_SHAPE, E_ALIGN, E_ENUM, E_ALIAS, E_BIG, E_LAUNCH, -99, 5):
        s = mxb.mx_strerror(code)
        assert isinstance(s, str) and s
    assert mxb.mx_strerror(-99) == "unknown libmx error"


@pytest.mark.parametrize("fmt,bpe", [("e4m3", 8.25), ("e5m2", 8.25), ("e2m1", 4.25), ("e2m3", 6.25),
                                     ("e3m2", 6.25), ("int8", 8.25)])
def test_plane_bytes(fmt, bpe):
    # "MXFP4 と NVFP4 は何が違うのか調べてみた" §2: 4.25 / 6.25 / 8.25 bits per element and plane
    for shape in [(16384, 4096), (14336, 4096), (64, 4096, 14336), (32, 32)]:
        n = 1
        for v in shape:
            n *= v
        for axis, planes in (("row", 1), ("col", 1), ("both", 2)):
            cb, sb = mxb.mx_plane_bytes(fmt, shape, axis)
            assert (cb + sb) * 8 / n == bpe * planes
            assert sb == planes * n // 32


def test_plane_bytes_errors(lib):
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    pb = lambda fmt, shape, axis, c=ctypes.byref(cb), s=ctypes.byref(sb): lib.mx_plane_bytes(fmt, MxShape(*shape),
                                                                                            axis, c, s)
    assert pb(0, (1, 4, 33), 1) == E_SHAPE                 # row blocks: cols % 32
    assert pb(0, (1, 4, 32), 2) == E_SHAPE                 # column blocks: rows % 32
    assert pb(0, (1, 32, 36), 2) == MX_OK and cb.value == 32 * 36 and sb.value == 36
    assert pb(0, (1, 4, 32), 1) == MX_OK and cb.value == 128 and sb.value == 4
    assert pb(2, (2, 64, 32), 3) == MX_OK and cb.value == 2 * 2 * 64 * 16 and sb.value == 2 * 2 * 64
    assert pb(0, (0, 4, 32), 1) == E_SHAPE
    assert pb(7, (1, 4, 32), 1) == E_ENUM
    assert pb(0, (1, 4, 32), 0) == E_ENUM
    assert pb(0, (1, 4, 32), 4) == E_ENUM
    assert pb(0, (1, 4, 32), 1, c=None) == E_NULL


# Fake, well-aligned, non-overlapping addresses: never dereferenced, because
# every call below fails validation first.
X, RC, RS, CC, CS, Y = (0x10000000 * k for k in range(1, 7))


def q(lib, x=X, dt=1, shape=(1, 64, 64), fmt=0, mode=0, axis=3, rc=RC, rs=RS, cc=CC, cs=CS):
    v = lambda p: ctypes.c_void_p(p)
    return lib.mx_quantize(v(x), dt, MxShape(*shape), fmt, mode, axis, v(rc), v(rs), v(cc), v(cs), None)


def test_quantize_argument_errors(lib):
    assert q(lib, fmt=6) == E_ENUM
    assert q(lib, fmt=-1) == E_ENUM
    assert q(lib, mode=2) == E_ENUM
    assert q(lib, dt=2) == E_ENUM
    assert q(lib, axis=0) == E_ENUM
    assert q(lib, axis=4) == E_ENUM
    assert q(lib, x=0) == E_NULL
    assert q(lib, rc=0) == E_NULL
    assert q(lib, cs=0) == E_NULL
    assert q(lib, axis=1) == E_NULL                    # column pointers must be NULL for row-only
    assert q(lib, axis=1, cc=0, cs=0, shape=(1, 64, 48)) == E_SHAPE
    assert q(lib, shape=(1, 64, 48)) == E_SHAPE        # row blocks of both copies: cols % 32
    assert q(lib, shape=(1, 48, 64)) == E_SHAPE        # column blocks need rows % 32 == 0
    # a column-only cast needs whole 16-byte row vectors only: cols % 8 (BF16), cols % 4 (FP32);
    # accepted shapes are shown by the alias check after the shape check failing
    assert q(lib, axis=2, rc=0, rs=0, shape=(1, 64, 36)) == E_SHAPE
    assert q(lib, axis=2, rc=0, rs=0, shape=(1, 64, 40), cc=X + 1024) == E_ALIAS
    assert q(lib, axis=2, rc=0, rs=0, dt=0, shape=(1, 64, 34)) == E_SHAPE
    assert q(lib, axis=2, rc=0, rs=0, dt=0, shape=(1, 64, 36), cc=X + 1024) == E_ALIAS
    assert q(lib, shape=(0, 64, 64)) == E_SHAPE
    assert q(lib, shape=(1, -32, 64)) == E_SHAPE
    assert q(lib, shape=(1, 1 << 40, 1 << 40)) == E_SHAPE
    assert q(lib, x=X + 8) == E_ALIGN
    assert q(lib, rc=RC + 4) == E_ALIGN
    assert q(lib, cc=CC + 1) == E_ALIGN
    assert q(lib, rc=X + 1024) == E_ALIAS              # row codes inside the input
    assert q(lib, cs=RS) == E_ALIAS                    # two outputs on one buffer


def test_dequantize_argument_errors(lib):
    v = lambda p: ctypes.c_void_p(p)
    dq = lambda c=CC, s=CS, fmt=0, shape=(1, 64, 64), dt=0, y=Y: lib.mx_dequantize(
        v(c), v(s), fmt, MxShape(*shape), dt, v(y), None)
    assert dq(fmt=9) == E_ENUM
    assert dq(dt=5) == E_ENUM
    assert dq(c=0) == E_NULL
    assert dq(s=0) == E_NULL
    assert dq(y=0) == E_NULL
    assert dq(shape=(1, 64, 40)) == E_SHAPE
    assert dq(shape=(1, 0, 64)) == E_SHAPE
    assert dq(c=CC + 8) == E_ALIGN
    assert dq(c=CC + 4, fmt=2) == E_ALIGN                # E2M1 codes: 8-byte aligned
    assert dq(c=CC + 2, fmt=3) == E_ALIGN                # E2M3 codes: 4-byte aligned
    assert dq(c=CC + 8, fmt=5) == E_ALIGN                # INT8 codes: 16-byte aligned
    assert dq(y=Y + 4) == E_ALIGN
    assert dq(y=CC + 16) == E_ALIAS


def test_python_binding_rejects_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        mxb.mx_quantize(torch.zeros(32, 32, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        mxb.mx_dequantize(torch.zeros(32, dtype=torch.uint8), torch.zeros(1, dtype=torch.uint8), "e4m3", (1, 32))


def test_python_binding_checks_every_buffer():
    """The binding checks each tensor against the sizes its shape and format
    imply before anything reaches the C ABI (which trusts them). With CPU
    tensors, a correct set of buffers gets as far as the GPU check."""
    import torch
    u8 = lambda n: torch.zeros(n, dtype=torch.uint8)
    f32 = lambda n: torch.zeros(n, dtype=torch.float32)

    def raises(fn, text):
        with pytest.raises(ValueError) as e:
            fn()
        assert text in str(e.value), str(e.value)
    gpu = "needs GPU"
    x = torch.zeros((64, 64), dtype=torch.bfloat16)
    # mx_quantize: caller-given planes
    ok = {"row_codes": u8(4096), "row_scales": u8(128), "col_codes": u8(4096), "col_scales": u8(128)}
    raises(lambda: mxb.mx_quantize(x, "e4m3", out=ok), gpu)
    raises(lambda: mxb.mx_quantize(x, "e4m3", out=dict(ok, row_codes=u8(4095))), "row_codes holds 4095")
    raises(lambda: mxb.mx_quantize(x, "e2m1", out=dict(ok)), "row_codes holds 4096")     # E2M1 needs 2048
    raises(lambda: mxb.mx_quantize(x, "e4m3", out=dict(ok, col_scales=f32(32))), "dtype")
    raises(lambda: mxb.mx_quantize(x, "e4m3", out=dict(ok, col_codes=u8(8192)[::2])), "contiguous")
    raises(lambda: mxb.mx_quantize(x, "e4m3", block="32x32", out=dict(ok)), "row_scales holds 128")
    raises(lambda: mxb.mx_quantize(x.to(torch.float16)), "bfloat16 or float32")
    raises(lambda: mxb.mx_quantize(x.t()), "contiguous")
    # mx_dequantize
    raises(lambda: mxb.mx_dequantize(u8(4096), u8(128), "e4m3", (64, 64)), gpu)
    raises(lambda: mxb.mx_dequantize(u8(4096), u8(127), "e4m3", (64, 64)), "scales holds 127")
    raises(lambda: mxb.mx_dequantize(u8(4096), u8(128), "e2m1", (64, 64)), "codes holds 4096")
    raises(lambda: mxb.mx_dequantize(u8(4096), u8(128), "e4m3", (64, 64), "f32", out=f32(4095)), "out holds")
    raises(lambda: mxb.mx_dequantize(u8(4096), u8(128), "e4m3", (64, 64), "f32",
                                     out=torch.zeros(4096, dtype=torch.bfloat16)), "dtype")
    raises(lambda: mxb.mx_dequantize(u8(4096), u8(4), "e4m3", (64, 64), block="32x32"), gpu)
    raises(lambda: mxb.BoundDequantize(u8(4096), u8(128), "e4m3", (64, 64), f32(4000)), "y holds")
    raises(lambda: mxb.BoundQuantize(x, "e4m3", "floor", "row", {"row_codes": u8(4096)}), "exactly")
    raises(lambda: mxb.BoundQuantize(x, "e4m3", "floor", "row", {"row_codes": u8(4096), "row_scales": u8(64)}),
           "row_scales holds 64")
    # NVFP4
    nv = {"global_scale": f32(1), "row_codes": u8(2048), "row_scales": u8(256), "col_codes": u8(2048),
          "col_scales": u8(256)}
    raises(lambda: mxb.mx_quantize_nvfp4(x, out=dict(nv)), gpu)
    raises(lambda: mxb.mx_quantize_nvfp4(x, out=dict(nv, row_scales=u8(128))), "row_scales holds 128")
    raises(lambda: mxb.mx_quantize_nvfp4(x, global_scale=f32(2), out=dict(nv)), "global_scale holds 8")
    raises(lambda: mxb.mx_dequantize_nvfp4(u8(2048), u8(256), f32(1), (64, 64)), gpu)
    raises(lambda: mxb.mx_dequantize_nvfp4(u8(2048), u8(256), u8(4), (64, 64)), "dtype")
    raises(lambda: mxb.mx_dequantize_nvfp4(u8(2048), u8(255), f32(1), (64, 64)), "scales holds 255")
    # FP4-in-FP8 requantization and the one-pass QAT step
    rq = {"e4m3": u8(4096), "block_scale": f32(1), "e4m3_t": u8(4096), "block_scale_t": f32(1), "spread": u8(1)}
    raises(lambda: mxb.mx_requant_fp4_fp8(u8(2048), u8(128), (64, 64), "both", out=dict(rq)), gpu)
    raises(lambda: mxb.mx_requant_fp4_fp8(u8(2048), u8(64), (64, 64), "both", out=dict(rq)), "scales holds 64")
    raises(lambda: mxb.mx_requant_fp4_fp8(u8(2048), u8(128), (64, 64), "both", out=dict(rq, block_scale=f32(2))),
           "block_scale holds 8")
    raises(lambda: mxb.mx_quantize_fp4_fp8(x, out=dict(rq, fp4_codes=u8(2047))), "fp4_codes holds 2047")
    raises(lambda: mxb.mx_quantize_fp4_fp8(x, out=dict(rq, e4m3_t=u8(4096).view(64, 64).t())), "contiguous")
    raises(lambda: mxb.mx_quantize_fp4_fp8(x, out=dict(rq)), gpu)


def qx(lib, opts=None, x=X, dt=1, shape=(1, 64, 64), fmt=0, mode=0, axis=3, rc=RC, rs=RS, cc=CC, cs=CS):
    v = lambda p: ctypes.c_void_p(p)
    o = ctypes.byref(opts) if opts is not None else None
    return lib.mx_quantize_ex(v(x), dt, MxShape(*shape), fmt, mode, axis, o, v(rc), v(rs), v(cc), v(cs), None)


def test_quantize_ex_argument_errors(lib):
    O = mxb.MxQuantOpts
    assert qx(lib, O(2, 0, 0)) == E_ENUM                 # unknown rounding
    assert qx(lib, O(0, 2, 0)) == E_ENUM                 # unknown block shape
    assert qx(lib, O(1, 0, 5), fmt=9) == E_ENUM
    # 32x32 blocks need rows % 32 == 0 even for the row copy alone
    assert qx(lib, O(0, 1, 0), axis=1, cc=0, cs=0, shape=(1, 48, 64)) == E_SHAPE
    # 1x32 blocks accept 48 rows for the row copy: the alias check after it fails
    assert qx(lib, O(0, 0, 0), axis=1, cc=0, cs=0, shape=(1, 48, 64), rc=X + 1024) == E_ALIAS
    assert qx(lib, O(1, 1, 0), rc=X + 1024) == E_ALIAS
    # a 32x32 scale plane is batch*rows*cols/1024 bytes: for 64 x 2^22 elements that is
    # 256 KiB, so a column scale plane right after it does not overlap (then the
    # cols >= 2^22 check fails), while the 8 MiB of 1x32 row scales would overlap it
    G = 1 << 32
    big = dict(shape=(1, 64, 1 << 22), x=G, rc=2 * G, rs=3 * G, cc=4 * G, cs=3 * G + (1 << 18), axis=3)
    assert qx(lib, O(0, 1, 0), **big) == E_BIG
    assert qx(lib, O(0, 0, 0), **big) == E_ALIAS
    assert qx(lib, O(1, 1, 0), x=0) == E_NULL
    assert qx(lib, O(1, 0, 0), x=X + 8) == E_ALIGN


def test_dequantize_ex_argument_errors(lib):
    v = lambda p: ctypes.c_void_p(p)
    dq = lambda block=1, c=CC, s=CS, fmt=0, shape=(1, 64, 64), dt=0, y=Y: lib.mx_dequantize_ex(
        v(c), v(s), fmt, MxShape(*shape), block, dt, v(y), None)
    assert dq(block=2) == E_ENUM
    assert dq(shape=(1, 48, 64)) == E_SHAPE               # 32x32 blocks: rows % 32
    assert dq(shape=(1, 64, 40)) == E_SHAPE
    assert dq(c=0) == E_NULL
    assert dq(y=CC + 16) == E_ALIAS
    assert dq(c=CC + 2, fmt=3) == E_ALIGN


def test_nvfp4_argument_errors(lib):
    v = lambda p: ctypes.c_void_p(p)
    G = 0x70000000

    def nq(x=X, dt=1, shape=(1, 64, 64), axis=3, gs=G, given=0, rc=RC, rs=RS, cc=CC, cs=CS):
        return lib.mx_quantize_nvfp4(v(x), dt, MxShape(*shape), axis, v(gs), given, v(rc), v(rs), v(cc), v(cs), None)
    assert nq(dt=3) == E_ENUM
    assert nq(axis=0) == E_ENUM
    assert nq(given=2) == E_ENUM
    assert nq(gs=0) == E_NULL
    assert nq(axis=1) == E_NULL
    assert nq(shape=(1, 64, 40)) == E_SHAPE                      # cols % 16
    assert nq(shape=(1, 40, 64)) == E_SHAPE                      # rows % 16 with a column copy
    # the row copy alone accepts 40 rows: the alias check after it fails
    assert nq(shape=(1, 40, 64), axis=1, cc=0, cs=0, rc=X + 64) == E_ALIAS
    assert nq(gs=G + 2) == E_ALIGN
    assert nq(x=X + 8) == E_ALIGN
    assert nq(gs=RS) == E_ALIAS
    assert nq(shape=(70000, 16, 16)) == E_BIG

    def nd(c=CC, s=CS, gs=G, shape=(1, 64, 64), dt=0, y=Y):
        return lib.mx_dequantize_nvfp4(v(c), v(s), v(gs), MxShape(*shape), dt, v(y), None)
    assert nd(dt=7) == E_ENUM
    assert nd(gs=0) == E_NULL
    assert nd(shape=(1, 64, 24)) == E_SHAPE
    assert nd(c=CC + 4) == E_ALIGN
    assert nd(y=CC + 16) == E_ALIAS


def test_requant_argument_errors(lib):
    """mx_requant_fp4_fp8: every case fails validation (addresses 4 GiB apart)."""
    v = lambda p: ctypes.c_void_p(p)
    G = 1 << 32
    C_, S_, F_, B_, FT, BT, SP = (G * k for k in range(1, 8))

    def rq(c=C_, s=S_, shape=(1, 64, 64), axis=3, f=F_, b=B_, ft=FT, bt=BT, sp=SP):
        return lib.mx_requant_fp4_fp8(v(c), v(s), MxShape(*shape), axis, v(f), v(b), v(ft), v(bt), v(sp), None)
    assert rq(axis=0) == E_ENUM
    assert rq(axis=4) == E_ENUM
    assert rq(c=0) == E_NULL
    assert rq(s=0) == E_NULL
    assert rq(f=0) == E_NULL                                     # row axis without its codes
    assert rq(axis=1) == E_NULL                                  # column planes given without the column axis
    assert rq(axis=2, bt=0) == E_NULL
    assert rq(shape=(1, 64, 48)) == E_SHAPE                      # cols % 32
    assert rq(shape=(0, 64, 64)) == E_SHAPE
    assert rq(shape=(1, 40, 64)) == E_SHAPE                      # rows % 16 with the transposed copy
    # the row copy alone accepts 40 rows: the alias check after it fails
    assert rq(shape=(1, 40, 64), axis=1, ft=0, bt=0, f=C_ + 16) == E_ALIAS
    assert rq(c=C_ + 8) == E_ALIGN
    assert rq(f=F_ + 8) == E_ALIGN
    assert rq(ft=FT + 8) == E_ALIGN
    assert rq(b=B_ + 2) == E_ALIGN
    assert rq(sp=C_ + 4) == E_ALIAS                              # spread overlaps the codes
    assert rq(bt=F_ + 16) == E_ALIAS
    assert rq(shape=(1, 1, 1 << 22), axis=1, ft=0, bt=0) == E_BIG
    assert rq(shape=(1, 1 << 23, 32)) == E_BIG                   # transposed rows too long


def test_quantize_fp4_fp8_argument_errors(lib):
    """mx_quantize_fp4_fp8: every case fails validation (addresses 4 GiB apart)."""
    v = lambda p: ctypes.c_void_p(p)
    G = 1 << 32
    X_, C_, S_, F_, B_, FT, BT, SP = (G * k for k in range(1, 9))

    def qq(x=X_, dt=0, shape=(1, 64, 64), mode=0, axis=3, c=C_, s=S_, f=F_, b=B_, ft=FT, bt=BT, sp=SP):
        return lib.mx_quantize_fp4_fp8(v(x), dt, MxShape(*shape), mode, axis, v(c), v(s), v(f), v(b), v(ft), v(bt),
                                       v(sp), None)
    assert qq(dt=2) == E_ENUM
    assert qq(mode=2) == E_ENUM
    assert qq(axis=0) == E_ENUM
    assert qq(x=0) == E_NULL
    assert qq(s=0) == E_NULL                                     # MXFP4 codes without their scales
    assert qq(axis=1) == E_NULL                                  # column planes without the column axis
    assert qq(shape=(1, 64, 48)) == E_SHAPE
    assert qq(shape=(1, 40, 64)) == E_SHAPE
    # no MXFP4 plane and the row copy alone accept 40 rows: the alias check after it fails
    assert qq(shape=(1, 40, 64), axis=1, c=0, s=0, ft=0, bt=0, f=X_ + 16) == E_ALIAS
    assert qq(x=X_ + 8) == E_ALIGN
    assert qq(c=C_ + 4) == E_ALIGN
    assert qq(c=X_ + 64) == E_ALIAS                              # MXFP4 codes over the weights
    assert qq(shape=(1, 1, 1 << 22), axis=1, ft=0, bt=0) == E_BIG


def test_copy_argument_errors(lib):
    """mx_copy_nt (the plain copy used as the bandwidth ceiling): every error
    path returns before any HIP call."""
    v = lambda p: ctypes.c_void_p(p)
    cp = lambda src=X, dst=Y, n=4096: lib.mx_copy_nt(v(src), v(dst), n, None)
    assert cp(src=0) == E_NULL
    assert cp(dst=0) == E_NULL
    assert cp(n=0) == E_SHAPE
    assert cp(n=-16) == E_SHAPE
    assert cp(n=4100) == E_SHAPE
    assert cp(src=X + 8) == E_ALIGN
    assert cp(dst=Y + 4) == E_ALIGN
    assert cp(dst=X + 1024) == E_ALIAS
    assert cp(src=Y + 2048) == E_ALIAS


def test_header_is_plain_c(tmp_path):
    """include/libmx.h is a C header: a strict C99 program includes it, links
    against libmx.so and makes host-side calls (sizes and error paths only)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "use_libmx.c"
    src.write_text(
        '#include "libmx.h"\n'
        "int main(void) {\n"
        "  mx_shape s = {1, 32, 64};\n"
        "  size_t code = 0, scale = 0;\n"
        "  if (mx_plane_bytes(MX_E2M1, s, MX_AXIS_ROW, &code, &scale) != MX_OK) return 1;\n"
        "  if (code != 1024 || scale != 64) return 2;\n"
        "  if (mx_plane_bytes(MX_E4M3, s, MX_AXIS_BOTH, &code, &scale) != MX_OK) return 5;\n"
        "  if (code != 4096 || scale != 128) return 6;\n"
        "  if (mx_quantize(0, MX_BF16, s, MX_E4M3, MX_SCALE_FLOOR, MX_AXIS_BOTH, 0, 0, 0, 0, 0) != MX_ERR_NULL) return 3;\n"
        "  if (mx_copy_nt(0, 0, 16, 0) != MX_ERR_NULL) return 4;\n"
        "  return mx_strerror(MX_ERR_ALIGN)[0] == 0;\n"
        "}\n")
    libdir = os.path.dirname(mxb.lib_path())
    exe = tmp_path / "use_libmx"
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
                        str(src), "-L", libdir, "-lmx", f"-Wl,-rpath,{libdir}", "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert subprocess.run([str(exe)]).returncode == 0
