// Device-side building blocks of the MX cast for gfx950 (CDNA4).
//
// Formats (the element layouts the pages fix, "MXFP4 と NVFP4 は何が違うのか調べてみた"
// §1-§2; FP8 bit layouts per the OCP 8-bit float definitions that article cites;
// the MXFP6 and MXINT8 rows of its §2 family table read as the OCP elements):
//   E4M3: max 448 = 1.75 * 2^8, no Inf, NaN = S.1111.111
//   E5M2: max 57344 = 1.75 * 2^15, IEEE-style Inf / NaN
//   E2M1: max 6 = 1.5 * 2^2, no Inf, no NaN
//   E2M3: bias 1, max 7.5 = 1.875 * 2^2; E3M2: bias 3, max 28 = 1.75 * 2^4;
//         both without Inf or NaN, sign in bit 5
//   INT8: two's-complement k read as k / 64, max 127/64 (emax 0), clipped
//         symmetrically to +-127
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
// E2M3 and E3M2 have no conversion of their own that takes two elements at a
// time, so they go through the FP8 format with the same mantissa width (the
// "carrier"): E2M3's grid is E4M3's subnormals and binades 2^-6..2^-4 moved
// up by 2^6, E3M2's is E5M2's subnormals and binades 2^-14..2^-8 moved up by
// 2^12. Dividing by 2^(e + shift) instead of 2^e therefore rounds exactly as
// the 6-bit format would, and the carrier code's low 5 bits are the 6-bit
// magnitude. INT8 is rounded in FP32 arithmetic (see int8_bits).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_enums.h"

namespace mx {

typedef short short2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));

// Per-format constants. emax = largest binade of the element format; the
// round-up rule adds one to the floor exponent when the block max's
// significand exceeds max / 2^emax (1.75 for the FP8 formats and E3M2, 1.5 for
// E2M1, 1.875 for E2M3, 1.984375 for INT8). bits = code bits in memory.
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
template <> struct FmtC<kE2M3> {
  static constexpr int emax = 2, bits = 6;
  static constexpr uint32_t thr_bf16 = 0x70, thr_f32 = 0x700000;
  static constexpr uint32_t nan_fill = 0u;            // no NaN code
  static constexpr int carrier = kE4M3, shift = 6;
};
template <> struct FmtC<kE3M2> {
  static constexpr int emax = 4, bits = 6;
  static constexpr uint32_t thr_bf16 = 0x60, thr_f32 = 0x600000;
  static constexpr uint32_t nan_fill = 0u;
  static constexpr int carrier = kE5M2, shift = 12;
};
template <> struct FmtC<kInt8> {
  static constexpr int emax = 0, bits = 8;
  static constexpr uint32_t thr_bf16 = 0x7E, thr_f32 = 0x7E0000;
  static constexpr uint32_t nan_fill = 0u;
};

template <int F> constexpr bool kIsFp6 = (F == kE2M3 || F == kE3M2);
// Codes are formed one per byte (E2M1: one per nibble); 6-bit codes are
// packed from bytes just before they are stored.
template <int F> constexpr int kRegBits = (F == kE2M1) ? 4 : 8;

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
// clamped below at 0 (2^-127); zero and subnormal maxima land there. With
// emax 0 (INT8) two more cases exist: the round-up step can pass 2^127 (it is
// clamped at code 254), and a subnormal block max 0.m * 2^-126 needs code 1
// only above max * 2^-127 = 0.9921875 * 2^-126, a different mantissa threshold
// (never reached by BF16's 7-bit subnormals).
template <int F, int M, bool BF16>
__device__ __forceinline__ uint32_t scale_code(uint32_t amag) {
  constexpr int mb = InC<BF16>::man_bits;
  constexpr uint32_t thr = BF16 ? FmtC<F>::thr_bf16 : FmtC<F>::thr_f32;
  int k = int(amag >> mb) - FmtC<F>::emax;
  if constexpr (M == kRoundUp) {
    uint32_t t = thr;
    if constexpr (FmtC<F>::emax == 0) t = (amag >> mb) == 0 ? (BF16 ? 0x7Fu : 0x7F0000u) : thr;
    k += ((amag & ((1u << mb) - 1u)) > t) ? 1 : 0;
  }
  k = k < 0 ? 0 : k;
  if constexpr (FmtC<F>::emax == 0 && M == kRoundUp) k = k > 254 ? 254 : k;
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

__device__ __forceinline__ float bf16_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t p) { return __uint_as_float(p & 0xFFFF0000u); }

// Carrier FP8 bytes -> 6-bit codes, one per byte, sign in bit 5. Under the
// floor rule the scaled block max is below 2^(emax+1), which the carrier can
// round up to exactly 2^(emax+1) (magnitude code 0x20) but never beyond: that
// one code saturates to 0x1F (+-max). Under the round-up rule nothing exceeds max.
template <int M>
__device__ __forceinline__ uint32_t fp6_from_carrier(uint32_t c) {
  uint32_t mag = c & 0x7F7F7F7Fu;
  if constexpr (M == kFloor) mag -= (mag >> 5) & 0x01010101u;
  return mag | ((c >> 2) & 0x20202020u);
}

// FP6 codes of two pairs of values (a0, a1, b0, b1 in element order) in one
// dword. The carrier's scale operand holds at most code 254 (2^127); blocks
// whose code + shift goes beyond it divide by the remaining 2^j in FP32 first.
// Such blocks have e >= 116, so every element that can round to a nonzero
// code (|x| >= 2^(e-5)) stays an FP32 normal and the division is exact; the
// others keep their sign and still round to zero.
template <int F, int M>
__device__ __forceinline__ uint32_t fp6_encode4_f32(float f0, float f1, float f2, float f3, uint32_t code) {
  constexpr int CF = FmtC<F>::carrier;
  constexpr uint32_t SH = FmtC<F>::shift;
  uint32_t kc = code + SH;
  if (code > 254u - SH) {
    const int j = int(kc) - 254;
    f0 = __builtin_ldexpf(f0, -j); f1 = __builtin_ldexpf(f1, -j);
    f2 = __builtin_ldexpf(f2, -j); f3 = __builtin_ldexpf(f3, -j);
    kc = 254u;
  }
  const float sc = scale_operand(kc);
  uint32_t c = cvt2_f32<CF, false>(0u, f0, f1, sc);
  c = cvt2_f32<CF, true>(c, f2, f3, sc);
  return code == 0xFFu ? FmtC<F>::nan_fill : fp6_from_carrier<M>(c);
}

// Same for two BF16 pairs; the common case converts BF16 directly.
template <int F, int M>
__device__ __forceinline__ uint32_t fp6_encode4_bf16(uint32_t p0, uint32_t p1, uint32_t code) {
  constexpr int CF = FmtC<F>::carrier;
  constexpr uint32_t SH = FmtC<F>::shift;
  if (code <= 254u - SH) {
    const float sc = scale_operand(code + SH);
    uint32_t c = cvt2_bf16<CF, false>(0u, p0, sc);
    c = cvt2_bf16<CF, true>(c, p1, sc);
    return fp6_from_carrier<M>(c);
  }
  return fp6_encode4_f32<F, M>(bf16_lo(p0), bf16_hi(p0), bf16_lo(p1), bf16_hi(p1), code);
}

// INT8: k = RNE(x * 2^(6 - e)) clipped to +-127. The FMA x * 2^(6-e) + 1.5 * 2^23
// is one rounding to an integer (the sum's ulp is 1 for |k| < 2^22, and its
// even/odd parity is k's), leaving k in the low bits of the result; the clip is
// an integer median on those bit patterns, and the low byte is k in two's
// complement. 2^(6-e) = 2^(133-code) is an FP32 normal for code >= 6; smaller
// codes (block max < 2^-121) first scale the inputs up by 2^127, exactly.
constexpr float kMagic = 12582912.0f;
constexpr int kMagicBits = 0x4B400000;

__device__ __forceinline__ uint32_t int8_bits(float f, float mul) {
  const int b = int(__float_as_uint(__builtin_fmaf(f, mul, kMagic)));
  return uint32_t(min(max(b, kMagicBits - 127), kMagicBits + 127));
}
// Low bytes of four dwords -> one dword, a in byte 0.
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_amdgcn_perm(b, a, 0x0C0C0400u) | __builtin_amdgcn_perm(d, c, 0x04000C0Cu);
}
__device__ __forceinline__ uint32_t int8_encode4(float f0, float f1, float f2, float f3, uint32_t code) {
  const bool tiny = code < 6u;
  const float pre = tiny ? 0x1p127f : 1.0f;
  const float mul = __uint_as_float((tiny ? 133u - code : 260u - code) << 23);
  const uint32_t w = pack_low_bytes(int8_bits(f0 * pre, mul), int8_bits(f1 * pre, mul),
                                    int8_bits(f2 * pre, mul), int8_bits(f3 * pre, mul));
  return code == 0xFFu ? FmtC<kInt8>::nan_fill : w;
}

// Four BF16 pairs straight from their bits, for block codes >= 8. A BF16 dot
// product with one zero weight gives x * 2^(133 - code) exactly (a BF16 value
// times a power of two that BF16 holds), and adding the magic constant rounds
// once to the nearest integer, as the FMA in int8_bits does. For code >= 8, a
// subnormal input scales below 0.5 and gives 0 whether or not the unit flushes
// it. An Inf or NaN partner in the other half of a pair poisons the sum, but
// such a block has code 0xFF and is overwritten.
__device__ __forceinline__ uint32_t int8_from_dot(uint32_t p, uint32_t wbits) {
  const float r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p), __builtin_bit_cast(bf16x2, wbits),
                                                  kMagic, false);
  const int b = int(__float_as_uint(r));
  return uint32_t(min(max(b, kMagicBits - 127), kMagicBits + 127));
}
__device__ __forceinline__ uint2 int8_encode8_bf16(uint32_t p0, uint32_t p1, uint32_t p2, uint32_t p3,
                                                   uint32_t code) {
  // a block code below 8 anywhere in the wave (block max < 2^-119) takes the
  // general path for the whole wave
  if (__builtin_amdgcn_ballot_w64(code < 8u) != 0) {
    return make_uint2(int8_encode4(bf16_lo(p0), bf16_hi(p0), bf16_lo(p1), bf16_hi(p1), code),
                      int8_encode4(bf16_lo(p2), bf16_hi(p2), bf16_lo(p3), bf16_hi(p3), code));
  }
  const uint32_t mb = (260u - code) << 7;              // 2^(133 - code) as BF16 bits
  const uint32_t wl = mb, wh = mb << 16;               // weights (m, 0) and (0, m)
  const uint32_t x = pack_low_bytes(int8_from_dot(p0, wl), int8_from_dot(p0, wh), int8_from_dot(p1, wl),
                                    int8_from_dot(p1, wh));
  const uint32_t y = pack_low_bytes(int8_from_dot(p2, wl), int8_from_dot(p2, wh), int8_from_dot(p3, wl),
                                    int8_from_dot(p3, wh));
  return code == 0xFFu ? make_uint2(FmtC<kInt8>::nan_fill, FmtC<kInt8>::nan_fill) : make_uint2(x, y);
}

// Encode four BF16 pairs (p0..p3, element order p0.lo, p0.hi, p1.lo, ...).
// FP8 / FP6 / INT8: 8 codes, one per byte, in two dwords. FP4: 8 codes in one
// dword (.y unused).
template <int F, int M>
__device__ __forceinline__ uint2 encode8_bf16(uint32_t p0, uint32_t p1, uint32_t p2, uint32_t p3,
                                              uint32_t code) {
  const float sc = scale_operand(code);
  uint2 r;
  if constexpr (kIsFp6<F>) {
    r.x = fp6_encode4_bf16<F, M>(p0, p1, code);
    r.y = fp6_encode4_bf16<F, M>(p2, p3, code);
  } else if constexpr (F == kInt8) {
    r = int8_encode8_bf16(p0, p1, p2, p3, code);
  } else if constexpr (F == kE2M1) {
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

// Encode four FP32 values. FP8 / FP6 / INT8: one dword, a code per byte.
// FP4: low 16 bits.
template <int F, int M>
__device__ __forceinline__ uint32_t encode4_f32(float f0, float f1, float f2, float f3,
                                                uint32_t code) {
  if constexpr (kIsFp6<F>) {
    return fp6_encode4_f32<F, M>(f0, f1, f2, f3, code);
  } else if constexpr (F == kInt8) {
    return int8_encode4(f0, f1, f2, f3, code);
  } else {
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
}

// Four 6-bit codes held one per byte -> bits 23:0, element 0 in bits 5:0 (the
// codes form a little-endian bit stream).
__device__ __forceinline__ uint32_t pack6(uint32_t w) {
  const uint32_t h = (w & 0x003F003Fu) | ((w >> 2) & 0x0FC00FC0u);   // 12-bit pairs in each half
  return (h & 0xFFFu) | ((h >> 4) & 0xFFF000u);
}
// 16 byte-held 6-bit codes -> 12 packed bytes.
__device__ __forceinline__ uint3 pack6x16(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
  const uint32_t a = pack6(w0), b = pack6(w1), c = pack6(w2), d = pack6(w3);
  return make_uint3(a | (b << 24), (b >> 8) | (c << 16), (c >> 16) | (d << 8));
}
// 12 packed bytes -> 16 6-bit codes, one per byte.
__device__ __forceinline__ uint32_t unpack6(uint32_t g) {   // bits 23:0 -> 4 bytes
  const uint32_t h = (g & 0xFFFu) | ((g << 4) & 0x0FFF0000u);
  return (h & 0x003F003Fu) | ((h << 2) & 0x3F003F00u);
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
// quad_perm [1,2,3,0] and [3,0,1,2]: lane 4q reads lanes 4q+1 and 4q+3
constexpr int kDppQuadNext = 0x39, kDppQuadPrev = 0x93;

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
