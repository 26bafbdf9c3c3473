/* Host-only driver of the libmx C ABI for the sanitizer build
 * (AddressSanitizer and UndefinedBehaviorSanitizer over mx_api.cpp and
 * mx_grid.cpp, linked against the stub launchers of mx_api_stubs.cpp). Every
 * MX_ERR_* path of every entry point is taken, with out-of-range enum values
 * as a C caller may pass them; accepted calls check what reaches the
 * launchers (flags, geometry, seed), and a failing launcher must come back as
 * MX_ERR_LAUNCH. Exit status 0: all checks passed; a sanitizer finding aborts. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "libmx.h"

int stub_calls(void);
void stub_fail_launches(int fail);
unsigned stub_nblocks(void);
unsigned stub_cast_flags(void);
unsigned stub_cast_tiles_r(void);
unsigned stub_cast_tiles_c(void);
long long stub_cast_cols(void);
int stub_cast_has_row_codes(void);
unsigned stub_cast_seed_lo(void);
unsigned stub_cast_seed_hi(void);
unsigned stub_nv_flags(void);
unsigned stub_rq_tiles_r(void);
unsigned stub_rq_tiles_c(void);
unsigned stub_rq_total(void);
unsigned stub_rq_flags(void);
unsigned stub_flag(int which);

static int fails = 0;
#define CHECK(c)                                                    \
  do {                                                              \
    if (!(c)) {                                                     \
      fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #c);        \
      ++fails;                                                      \
    }                                                               \
  } while (0)

/* fake device addresses, 256 MiB apart: never dereferenced (the launchers are stubs) */
static void* A(int k) { return (void*)((uintptr_t)k << 28); }
static uint8_t* B(int k) { return (uint8_t*)A(k); }
static float* F(int k) { return (float*)A(k); }

static int q(mx_shape sh, int ax, void* x, void* rc, uint8_t* rs, void* cc, uint8_t* cs, const mx_quant_opts* o,
             int dt, int fmt) {
  return mx_quantize_ex(x, (mx_dtype)dt, sh, (mx_fmt)fmt, MX_SCALE_FLOOR, (mx_axis)ax, o, rc, rs, cc, cs, 0);
}

static int nq(mx_shape sh, int ax, float* gs, int given) {
  return mx_quantize_nvfp4(A(1), MX_BF16, sh, (mx_axis)ax, gs, given, (ax & 1) ? A(2) : 0, (ax & 1) ? B(3) : 0,
                           (ax & 2) ? A(4) : 0, (ax & 2) ? B(5) : 0, 0);
}

int main(void) {
  const mx_shape s = {1, 256, 512};
  size_t cb = 0, sb = 0;
  int e;

  /* ---- mx_plane_bytes ---- */
  CHECK(mx_plane_bytes(MX_E4M3, s, MX_AXIS_BOTH, &cb, &sb) == MX_OK && cb == 2 * 256 * 512 && sb == 2 * 256 * 16);
  CHECK(mx_plane_bytes(MX_E2M3, s, MX_AXIS_ROW, &cb, &sb) == MX_OK && cb == 256 * 512 * 3 / 4);
  CHECK(mx_plane_bytes((mx_fmt)9, s, MX_AXIS_ROW, &cb, &sb) == MX_ERR_ENUM);
  CHECK(mx_plane_bytes((mx_fmt)-1, s, MX_AXIS_ROW, &cb, &sb) == MX_ERR_ENUM);
  CHECK(mx_plane_bytes(MX_E4M3, s, (mx_axis)0, &cb, &sb) == MX_ERR_ENUM);
  CHECK(mx_plane_bytes(MX_E4M3, s, (mx_axis)1000, &cb, &sb) == MX_ERR_ENUM);
  CHECK(mx_plane_bytes(MX_E4M3, s, MX_AXIS_ROW, NULL, &sb) == MX_ERR_NULL);
  {
    const mx_shape r40 = {1, 256, 40}, c40 = {1, 40, 512}, huge = {INT64_MAX, INT64_MAX, 32};
    CHECK(mx_plane_bytes(MX_E4M3, r40, MX_AXIS_ROW, &cb, &sb) == MX_ERR_SHAPE);
    CHECK(mx_plane_bytes(MX_E4M3, c40, MX_AXIS_COL, &cb, &sb) == MX_ERR_SHAPE);
    CHECK(mx_plane_bytes(MX_E4M3, huge, MX_AXIS_ROW, &cb, &sb) == MX_ERR_SHAPE);
  }

  /* ---- mx_quantize / mx_quantize_ex ---- */
  {
    const mx_shape c48 = {1, 256, 48}, r48 = {1, 48, 512}, c36 = {1, 256, 36}, neg = {-1, 256, 512};
    const mx_shape over = {INT64_MAX / 2, 4, 32}, wide = {1, 32, (1 << 22) - 32}, too = {1, 32, 1 << 22};
    const mx_shape c40 = {1, 256, 40}, act = {1, 16384, 4096};
    mx_quant_opts bad_r, bad_b, sr;
    memset(&bad_r, 0, sizeof bad_r);
    bad_r.rounding = (mx_rounding)3;
    memset(&bad_b, 0, sizeof bad_b);
    bad_b.block = (mx_block)-7;
    sr.rounding = MX_ROUND_STOCHASTIC;
    sr.block = MX_BLOCK_32X32;
    sr.seed = 0x123456789ABCDEF0ull;
    CHECK(q(s, 3, NULL, A(2), B(3), A(4), B(5), NULL, MX_BF16, MX_E4M3) == MX_ERR_NULL);
    CHECK(q(s, 1, A(1), A(2), B(3), A(4), B(5), NULL, MX_BF16, MX_E4M3) == MX_ERR_NULL);
    CHECK(q(s, 3, A(1), A(2), B(3), A(4), B(5), NULL, 7, MX_E4M3) == MX_ERR_ENUM);
    CHECK(q(s, 3, A(1), A(2), B(3), A(4), B(5), NULL, MX_BF16, 6) == MX_ERR_ENUM);
    CHECK(q(s, 8, A(1), A(2), B(3), A(4), B(5), NULL, MX_BF16, MX_E4M3) == MX_ERR_ENUM);
    CHECK(q(c48, 3, A(1), A(2), B(3), A(4), B(5), NULL, MX_BF16, MX_E4M3) == MX_ERR_SHAPE);
    CHECK(q(r48, 3, A(1), A(2), B(3), A(4), B(5), NULL, MX_BF16, MX_E4M3) == MX_ERR_SHAPE);
    CHECK(q(c36, 2, A(1), NULL, NULL, A(4), B(5), NULL, MX_BF16, MX_E4M3) == MX_ERR_SHAPE);
    CHECK(q(neg, 3, A(1), A(2), B(3), A(4), B(5), NULL, MX_BF16, MX_E4M3) == MX_ERR_SHAPE);
    CHECK(q(over, 1, A(1), A(2), B(3), NULL, NULL, NULL, MX_BF16, MX_E4M3) == MX_ERR_SHAPE);
    CHECK(q(s, 3, B(1) + 8, A(2), B(3), A(4), B(5), NULL, MX_BF16, MX_E4M3) == MX_ERR_ALIGN);
    CHECK(q(s, 3, A(1), B(1) + 4096, B(3), A(4), B(5), NULL, MX_BF16, MX_E4M3) == MX_ERR_ALIAS);
    CHECK(q(wide, 1, A(1), A(4), B(7), NULL, NULL, NULL, MX_BF16, MX_E4M3) == MX_OK);   /* the row stream */
    CHECK(q(too, 1, A(1), A(4), B(7), NULL, NULL, NULL, MX_BF16, MX_E4M3) == MX_ERR_TOO_LARGE);
    CHECK(q(s, 3, A(1), A(2), B(3), A(4), B(5), &bad_r, MX_BF16, MX_E4M3) == MX_ERR_ENUM);
    CHECK(q(s, 3, A(1), A(2), B(3), A(4), B(5), &bad_b, MX_BF16, MX_E4M3) == MX_ERR_ENUM);

    e = stub_calls();
    CHECK(q(act, 3, A(1), A(2), B(3), A(4), B(5), NULL, MX_BF16, MX_E4M3) == MX_OK);
    CHECK(stub_calls() == e + 1 && stub_nblocks() == 128 * 16 && stub_cast_tiles_r() == 128 &&
          stub_cast_tiles_c() == 16);
    CHECK((stub_cast_flags() & stub_flag(0)) && (stub_cast_flags() & stub_flag(1)) &&
          (stub_cast_flags() & stub_flag(2)) && (stub_cast_flags() & stub_flag(3)));
    CHECK(q(c40, 2, A(1), NULL, NULL, A(4), B(5), NULL, MX_BF16, MX_E4M3) == MX_OK);
    CHECK(!stub_cast_has_row_codes() && stub_cast_cols() == 40 && stub_cast_tiles_c() == 1);
    CHECK(q(c36, 2, A(1), NULL, NULL, A(4), B(5), NULL, MX_F32, MX_E2M1) == MX_OK);
    CHECK(q(s, 3, A(1), A(2), B(3), A(4), B(5), &sr, MX_BF16, MX_E4M3) == MX_OK);
    CHECK(stub_cast_seed_lo() == 0x9ABCDEF0u && stub_cast_seed_hi() == 0x12345678u);
    stub_fail_launches(1);
    CHECK(q(s, 3, A(1), A(2), B(3), A(4), B(5), NULL, MX_BF16, MX_E4M3) == MX_ERR_LAUNCH);
    stub_fail_launches(0);
  }

  /* ---- mx_dequantize / mx_dequantize_ex ---- */
  {
    const mx_shape c20 = {1, 4, 20}, r48 = {1, 48, 64};
    CHECK(mx_dequantize(A(1), B(2), MX_E4M3, s, MX_F32, A(3), 0) == MX_OK);
    CHECK(mx_dequantize(NULL, B(2), MX_E4M3, s, MX_F32, A(3), 0) == MX_ERR_NULL);
    CHECK(mx_dequantize(A(1), B(2), (mx_fmt)-1, s, MX_F32, A(3), 0) == MX_ERR_ENUM);
    CHECK(mx_dequantize(A(1), B(2), MX_E4M3, s, (mx_dtype)2, A(3), 0) == MX_ERR_ENUM);
    CHECK(mx_dequantize(A(1), B(2), MX_E4M3, c20, MX_F32, A(3), 0) == MX_ERR_SHAPE);
    CHECK(mx_dequantize(B(1) + 4, B(2), MX_E2M1, s, MX_F32, A(3), 0) == MX_ERR_ALIGN);
    CHECK(mx_dequantize(A(1), B(2), MX_E4M3, s, MX_F32, B(1) + 64, 0) == MX_ERR_ALIAS);
    CHECK(mx_dequantize_ex(A(1), B(2), MX_E4M3, r48, MX_BLOCK_32X32, MX_F32, A(3), 0) == MX_ERR_SHAPE);
    CHECK(mx_dequantize_ex(A(1), B(2), MX_E4M3, s, (mx_block)9, MX_F32, A(3), 0) == MX_ERR_ENUM);
    stub_fail_launches(1);
    CHECK(mx_dequantize(A(1), B(2), MX_E4M3, s, MX_BF16, A(3), 0) == MX_ERR_LAUNCH);
    stub_fail_launches(0);
  }

  /* ---- NVFP4 ---- */
  {
    const mx_shape c24 = {1, 256, 24}, big = {70000, 16, 16};
    e = stub_calls();
    CHECK(nq(s, 3, F(6), 0) == MX_OK && stub_calls() == e + 2 && (stub_nv_flags() & stub_flag(4)));
    CHECK(nq(s, 3, F(6), 1) == MX_OK && stub_calls() == e + 3 && !(stub_nv_flags() & stub_flag(4)));
    CHECK(nq(s, 3, NULL, 0) == MX_ERR_NULL);
    CHECK(nq(s, 3, F(6), 2) == MX_ERR_ENUM);
    CHECK(nq(s, 0, F(6), 0) == MX_ERR_ENUM);
    CHECK(nq(c24, 1, F(6), 0) == MX_ERR_SHAPE);
    CHECK(nq(s, 3, (float*)(B(6) + 2), 0) == MX_ERR_ALIGN);
    CHECK(nq(s, 3, (float*)(B(3) + 4), 0) == MX_ERR_ALIAS);
    CHECK(nq(big, 1, F(6), 0) == MX_ERR_TOO_LARGE);
    stub_fail_launches(1);
    CHECK(nq(s, 3, F(6), 0) == MX_ERR_LAUNCH);
    stub_fail_launches(0);
    CHECK(mx_dequantize_nvfp4(A(1), B(2), F(3), s, MX_F32, A(4), 0) == MX_OK);
    CHECK(mx_dequantize_nvfp4(A(1), B(2), NULL, s, MX_F32, A(4), 0) == MX_ERR_NULL);
    CHECK(mx_dequantize_nvfp4(A(1), B(2), F(3), s, (mx_dtype)5, A(4), 0) == MX_ERR_ENUM);
    CHECK(mx_dequantize_nvfp4(A(1), B(2), F(3), c24, MX_F32, A(4), 0) == MX_ERR_SHAPE);
    CHECK(mx_dequantize_nvfp4(B(1) + 4, B(2), F(3), s, MX_F32, A(4), 0) == MX_ERR_ALIGN);
    CHECK(mx_dequantize_nvfp4(A(1), B(2), F(3), s, MX_F32, B(2) + 16, 0) == MX_ERR_ALIAS);
  }

  /* ---- FP4-in-FP8 ---- */
  {
    const mx_shape r40 = {1, 40, 64};
    CHECK(mx_requant_fp4_fp8(A(1), B(2), s, MX_AXIS_BOTH, B(3), F(4), B(5), F(6), B(7), 0) == MX_OK);
    CHECK(stub_rq_tiles_r() == 2 && stub_rq_tiles_c() == 2 && stub_rq_total() == 4 && (stub_rq_flags() & stub_flag(5)));
    CHECK(!(stub_rq_flags() & stub_flag(6)));
    {
      const mx_shape b4 = {4, 256, 512};
      CHECK(mx_requant_fp4_fp8(A(1), B(2), b4, MX_AXIS_BOTH, B(3), F(4), B(5), F(6), B(7), 0) == MX_OK);
      CHECK(stub_rq_total() == 16 && (stub_rq_flags() & stub_flag(6)));
    }
    CHECK(mx_requant_fp4_fp8(A(1), B(2), s, (mx_axis)5, B(3), F(4), B(5), F(6), B(7), 0) == MX_ERR_ENUM);
    CHECK(mx_requant_fp4_fp8(A(1), NULL, s, MX_AXIS_BOTH, B(3), F(4), B(5), F(6), B(7), 0) == MX_ERR_NULL);
    CHECK(mx_requant_fp4_fp8(A(1), B(2), r40, MX_AXIS_BOTH, B(3), F(4), B(5), F(6), B(7), 0) == MX_ERR_SHAPE);
    CHECK(mx_requant_fp4_fp8(A(1), B(2), s, MX_AXIS_BOTH, B(3) + 8, F(4), B(5), F(6), B(7), 0) == MX_ERR_ALIGN);
    CHECK(mx_requant_fp4_fp8(A(1), B(2), s, MX_AXIS_BOTH, B(3), F(4), B(5), F(6), B(1) + 8, 0) == MX_ERR_ALIAS);
    CHECK(mx_quantize_fp4_fp8(A(1), MX_F32, s, MX_SCALE_ROUNDUP, MX_AXIS_ROW, A(2), B(3), B(4), F(5), NULL, NULL,
                              NULL, 0) == MX_OK);
    CHECK(mx_quantize_fp4_fp8(A(1), MX_F32, s, MX_SCALE_ROUNDUP, MX_AXIS_ROW, A(2), NULL, B(4), F(5), NULL, NULL,
                              NULL, 0) == MX_ERR_NULL);
    CHECK(mx_quantize_fp4_fp8(A(1), MX_F32, s, (mx_scale_mode)4, MX_AXIS_ROW, A(2), B(3), B(4), F(5), NULL, NULL,
                              NULL, 0) == MX_ERR_ENUM);
    stub_fail_launches(1);
    CHECK(mx_requant_fp4_fp8(A(1), B(2), s, MX_AXIS_BOTH, B(3), F(4), B(5), F(6), B(7), 0) == MX_ERR_LAUNCH);
    stub_fail_launches(0);
  }

  /* ---- mx_copy_nt, mx_strerror, mx_version ---- */
  CHECK(mx_copy_nt(A(1), A(2), 4096, 0) == MX_OK);
  CHECK(mx_copy_nt(A(1), A(2), 4095, 0) == MX_ERR_SHAPE);
  CHECK(mx_copy_nt(A(1), B(1) + 16, 4096, 0) == MX_ERR_ALIAS);
  CHECK(mx_copy_nt(B(1) + 8, A(2), 4096, 0) == MX_ERR_ALIGN);
  CHECK(mx_copy_nt(NULL, A(2), 4096, 0) == MX_ERR_NULL);
  for (e = -9; e <= 1; ++e) CHECK(mx_strerror(e) != NULL && strlen(mx_strerror(e)) > 0);
  CHECK(mx_version() == 10700);

  if (fails) return 1;
  puts("mx_api host checks passed");
  return 0;
}
