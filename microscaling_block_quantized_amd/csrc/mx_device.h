// Device-side building blocks of the MX cast for gfx950 (CDNA4).
//
// Formats (the element layouts the pages fix, "MXFP4 と NVFP4 は何が違うのか調べてみた"
// §1-§2; FP8 bit layouts per the OCP 8-bit float definitions that article cites):
//   E4M3: max 448 = 1.75 * 2^8, no Inf, NaN = S.1111.111
//   E5M2: max 57344 = 1.75 * 2^15, IEEE-style Inf / NaN
//   E2M1: max 6 = 1.5 * 2^2, no Inf, no NaN
//   E8M0 scale: code k <-> 2^(k-127), 0xFF = NaN (same article, §2).
//
// The element encoders are the gfx950 scaled down-conversions
// (v_cvt_scalef32_pk_{fp8,bf8,fp4}_{bf16,f32}). Measured behaviour they rely on:
//   * the scale operand is an FP32 whose exponent field is used as an E8M0
//     code (field k divides the input by 2^(k-127); field 0 means 2^-127);
//   * rounding is round-to-nearest-even, including FP8 subnormals and the
//     sign of zero;
//   * the FP8 forms do not saturate: a magnitude beyond max becomes 0x7F
//     (E4M3 NaN) or 0x7C (E5M2 Inf); fix_overflow() turns those into +-max;
//   * the FP4 form saturates to +-6.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

enum Fmt : int { kE4M3 = 0, kE5M2 = 1, kE2M1 = 2 };
enum Mode : int { kFloor = 0, kRoundUp = 1 };
enum Axis : int { kRow = 1, kCol = 2, kBoth = 3 };

typedef short short2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));

// Per-format constants. emax = largest binade of the element format; the
// round-up rule adds one to the floor exponent when the block max's
// significand exceeds max / 2^emax (1.75 for the FP8 formats, 1.5 for E2M1).
template <int F> struct FmtC;
template <> struct FmtC<kE4M3> {
  static constexpr int emax = 8, bits = 8;
  static constexpr uint32_t thr_bf16 = 0x60, thr_f32 = 0x600000;
  static constexpr uint32_t nan_fill = 0x7F7F7F7Fu;   // every element NaN
  static constexpr uint32_t ovf_add = 0x01010101u;    // byte 0x7F -> carries into bit 7
};
template <> struct FmtC<kE5M2> {
  static constexpr int emax = 15, bits = 8;
  static constexpr uint32_t thr_bf16 = 0x60, thr_f32 = 0x600000;
  static constexpr uint32_t nan_fill = 0x7F7F7F7Fu;
  static constexpr uint32_t ovf_add = 0x04040404u;    // byte 0x7C -> carries into bit 7
};
template <> struct FmtC<kE2M1> {
  static constexpr int emax = 2, bits = 4;
  static constexpr uint32_t thr_bf16 = 0x40, thr_f32 = 0x400000;
  static constexpr uint32_t nan_fill = 0u;
  static constexpr uint32_t ovf_add = 0u;
};

// Input element types: BF16 is carried as raw 16-bit patterns.
template <bool BF16> struct InC;
template <> struct InC<true> {
  static constexpr int vec = 8;                       // elements per 16-byte load
  static constexpr int man_bits = 7;
  static constexpr uint32_t special = 0x7F80u;         // |x| bits >= this: Inf or NaN
};
template <> struct InC<false> {
  static constexpr int vec = 4;
  static constexpr int man_bits = 23;
  static constexpr uint32_t special = 0x7F800000u;
};

// E8M0 code of a block from the integer maximum of its magnitude bits.
// Integer order of |x| bit patterns puts NaN above Inf above every finite
// value, so one max finds both the block max and any special value.
//   FLOOR  : k = floor(log2 amax) - emax + 127 = exponent_field - emax
//   ROUNDUP: k + 1 when the significand of amax exceeds max / 2^emax
// clamped below at 0 (2^-127); zero and subnormal maxima land there.
template <int F, int M, bool BF16>
__device__ __forceinline__ uint32_t scale_code(uint32_t amag) {
  constexpr int mb = InC<BF16>::man_bits;
  constexpr uint32_t thr = BF16 ? FmtC<F>::thr_bf16 : FmtC<F>::thr_f32;
  int k = int(amag >> mb) - FmtC<F>::emax;
  if constexpr (M == kRoundUp) k += ((amag & ((1u << mb) - 1u)) > thr) ? 1 : 0;
  k = k < 0 ? 0 : k;
  return amag >= InC<BF16>::special ? 0xFFu : uint32_t(k);
}

__device__ __forceinline__ float scale_operand(uint32_t code) {
  return __uint_as_float(code << 23);
}

// FP8 results of magnitude 0x7F (E4M3) or 0x7C (E5M2) come only from
// overflow of finite inputs: step them down to +-max, byte-wise.
template <int F>
__device__ __forceinline__ uint32_t fix_overflow(uint32_t c) {
  uint32_t hit = (((c & 0x7F7F7F7Fu) + FmtC<F>::ovf_add) & 0x80808080u) >> 7;
  return c - hit;
}

__device__ __forceinline__ uint32_t bits_of(short2v v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ short2v s2_of(uint32_t v) { return __builtin_bit_cast(short2v, v); }
__device__ __forceinline__ bf16x2 b2_of(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

// Two BF16 (element 0 in the low half) -> two FP8 bytes in half W of `old`.
template <int F, bool W>
__device__ __forceinline__ uint32_t cvt2_bf16(uint32_t old, uint32_t pair, float sc) {
  if constexpr (F == kE4M3)
    return bits_of(__builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(s2_of(old), b2_of(pair), sc, W));
  else
    return bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(s2_of(old), b2_of(pair), sc, W));
}
template <int F, bool W>
__device__ __forceinline__ uint32_t cvt2_f32(uint32_t old, float a, float b, float sc) {
  if constexpr (F == kE4M3)
    return bits_of(__builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s2_of(old), a, b, sc, W));
  else
    return bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf8_f32(s2_of(old), a, b, sc, W));
}
// Two elements -> one E2M1 byte (element 0 in bits 3:0) at byte S of `old`.
template <int S>
__device__ __forceinline__ uint32_t cvt2_fp4_bf16(uint32_t old, uint32_t pair, float sc) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(old, b2_of(pair), sc, S);
}
template <int S>
__device__ __forceinline__ uint32_t cvt2_fp4_f32(uint32_t old, float a, float b, float sc) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, sc, S);
}

// Encode four BF16 pairs (p0..p3, element order p0.lo, p0.hi, p1.lo, ...).
// FP8: 8 codes in two dwords. FP4: 8 codes in one dword (.y unused).
template <int F, int M>
__device__ __forceinline__ uint2 encode8_bf16(uint32_t p0, uint32_t p1, uint32_t p2, uint32_t p3,
                                              uint32_t code) {
  const float sc = scale_operand(code);
  uint2 r;
  if constexpr (F == kE2M1) {
    uint32_t w = cvt2_fp4_bf16<0>(0u, p0, sc);
    w = cvt2_fp4_bf16<1>(w, p1, sc);
    w = cvt2_fp4_bf16<2>(w, p2, sc);
    w = cvt2_fp4_bf16<3>(w, p3, sc);
    r.x = code == 0xFFu ? FmtC<F>::nan_fill : w;
    r.y = 0;
  } else {
    uint32_t a = cvt2_bf16<F, false>(0u, p0, sc);
    a = cvt2_bf16<F, true>(a, p1, sc);
    uint32_t b = cvt2_bf16<F, false>(0u, p2, sc);
    b = cvt2_bf16<F, true>(b, p3, sc);
    if constexpr (M == kFloor) { a = fix_overflow<F>(a); b = fix_overflow<F>(b); }
    r.x = code == 0xFFu ? FmtC<F>::nan_fill : a;
    r.y = code == 0xFFu ? FmtC<F>::nan_fill : b;
  }
  return r;
}

// Encode four FP32 values. FP8: one dword. FP4: low 16 bits.
template <int F, int M>
__device__ __forceinline__ uint32_t encode4_f32(float f0, float f1, float f2, float f3,
                                                uint32_t code) {
  const float sc = scale_operand(code);
  uint32_t w;
  if constexpr (F == kE2M1) {
    w = cvt2_fp4_f32<0>(0u, f0, f1, sc);
    w = cvt2_fp4_f32<1>(w, f2, f3, sc);
  } else {
    w = cvt2_f32<F, false>(0u, f0, f1, sc);
    w = cvt2_f32<F, true>(w, f2, f3, sc);
    if constexpr (M == kFloor) w = fix_overflow<F>(w);
  }
  return code == 0xFFu ? FmtC<F>::nan_fill : w;
}

// max over the two 16-bit halves independently (v_pk_max_u16).
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}

// Cross-lane moves without LDS. DPP patterns act inside each 16-lane row:
// quad_perm [1,0,3,2] = lane ^ 1, [2,3,0,1] = lane ^ 2, row_half_mirror maps
// lane i of an 8-lane half to 7 - i, row_ror:n rotates the row by n lanes.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return __builtin_amdgcn_update_dpp(0u, v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppRor4 = 0x124, kDppRor8 = 0x128;

// gfx950 v_permlane{16,32}_swap with both operands equal: the two results
// hold, for every lane, its own value and the value of lane ^ 16 (resp. ^ 32).
__device__ __forceinline__ uint32_t max_xor16(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return max(uint32_t(r[0]), uint32_t(r[1]));
}
__device__ __forceinline__ uint32_t max_xor32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max(uint32_t(r[0]), uint32_t(r[1]));
}
__device__ __forceinline__ uint32_t pk_max_xor16(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return pk_max_u16(uint32_t(r[0]), uint32_t(r[1]));
}
__device__ __forceinline__ uint32_t pk_max_xor32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return pk_max_u16(uint32_t(r[0]), uint32_t(r[1]));
}
__device__ __forceinline__ uint32_t or_xor16(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return uint32_t(r[0]) | uint32_t(r[1]);
}

// Max over aligned groups of N lanes (N = 4 or 8) inside a 16-lane row.
template <int N>
__device__ __forceinline__ uint32_t group_max(uint32_t v) {
  v = max(v, dpp<kDppXor1>(v));
  v = max(v, dpp<kDppXor2>(v));
  if constexpr (N == 8) v = max(v, dpp<kDppHalfMirror>(v));
  return v;
}

}  // namespace mx
